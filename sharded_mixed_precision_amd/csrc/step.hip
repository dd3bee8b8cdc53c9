// Device side of the shard-local mixed-precision AdamW step for gfx950
// (MI355X): the kernels and the entry points that launch them.
//
// Pages cited: [DO] "Megatron-LM distrib_optimizer.py 源码精读";
// [ZL] "02 · ZeRO 显存账本与 Megatron DistributedOptimizer";
// [DS] "Megatron-LM与DeepSpeed的分布式训练源码里，模型和优化器到底是怎么切分的？".
//
// The step is bound by HBM bandwidth (about 1 flop per byte), so no matrix
// cores are involved.  Each pass streams the arena arrays once with 16-byte
// loads and stores: one 256-thread workgroup per 2048-element tile, 8
// consecutive elements per thread, grid-stride over the tiles (the fused
// reduce and the state copy of a large window in launches of kRangeTiles
// tiles).  Tiles that lie inside one param's shard (nearly all) take a
// branch-free path; tiles that hold a shard boundary, a 64-element alignment
// gap or the arena tail test each element against the few segments that
// overlap them (pass 2 of a large window with such tiles in k_apply_bnd).
//
// Arithmetic is IEEE fp32 in the order stated at adamw() below: the library
// is built with contraction off, correctly rounded sqrt and division, and
// denormals kept.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

#include "internal.h"

namespace dopt {

// ---- device records in the workspace -------------------------------------

struct DevState {  // persists across steps
    double scale, growth_factor, backoff_factor, min_scale;
    int64_t t;  // successful steps
    int64_t growth_tracker, hysteresis_tracker, growth_interval;
    float inv_scale;  // fp32(1 / scale): the unscale factor of the coming step
    int32_t kind, hysteresis, pad;
};
static_assert(sizeof(DevState) <= kWsStepRec - kWsState, "state record too large");

struct StepRec {  // scalars of the apply pass of the current step
    int32_t skip, clip_on;
    float inv_scale, clip;
    float decay[DOPT_MAX_HGROUPS], beta1[DOPT_MAX_HGROUPS], omb1[DOPT_MAX_HGROUPS];
    float beta2[DOPT_MAX_HGROUPS], omb2[DOPT_MAX_HGROUPS], eps[DOPT_MAX_HGROUPS];
    float step_size[DOPT_MAX_HGROUPS], sqrt_bc2[DOPT_MAX_HGROUPS];
};
static_assert(sizeof(StepRec) <= kWsStats - kWsStepRec, "step record too large");
static_assert(sizeof(dopt_stats) <= kWsRecord - kWsStats, "stats record too large");

struct Partial {
    double sumsq;
    unsigned long long zeros;
};
static_assert(sizeof(Partial) == 16, "partial record size");

struct Record {
    double sumsq, zeros;
};

struct FinalizeArgs {
    dopt_hparams hp[DOPT_MAX_HGROUPS];
    int32_t nh, pad;
    double max_norm;
};

struct InitArgs {
    DevState st;
};

// ---- element I/O -----------------------------------------------------------

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16-byte load; NT marks the line as streamed (read once), which lets the
// memory system keep it out of the caches.
template <bool NT>
__device__ __forceinline__ u32x4 ld16(const void *p) {
    if (NT) return __builtin_nontemporal_load(static_cast<const u32x4 *>(p));
    return *static_cast<const u32x4 *>(p);
}

// Tile-local buffer access (pass 2).  A resource descriptor covers one
// 2048-element tile of one stream: the tile base is wave-uniform and sits in
// scalar registers, so every stream of a tile shares one per-lane byte offset
// instead of holding a 64-bit address per lane.  The descriptor is raw
// (stride 0, range in bytes) with the 32-bit data format that untyped dword
// accesses take on this ISA; an access past the range would read zero and
// write nothing, and none is made.
constexpr int32_t kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void *tile_base, int32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(tile_base), 0, bytes, kRsrcWord3);
}
__device__ __forceinline__ u32x4 bld16(__amdgpu_buffer_rsrc_t r, int32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ void bst16(__amdgpu_buffer_rsrc_t r, int32_t off, u32x4 x) {
    __builtin_amdgcn_raw_buffer_store_b128(x, r, off, 0, 0);
}
__device__ __forceinline__ float bld4(__amdgpu_buffer_rsrc_t r, int32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void bst4(__amdgpu_buffer_rsrc_t r, int32_t off, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 0);
}

template <int DT>
struct Elem;

// The raw bytes of 8 consecutive elements (16-bit types use `lo` only).
// Kernels load raw packets first and convert after a scheduling barrier, so
// that all of a batch's loads are in flight before the first one is waited
// for.
struct Raw8 {
    u32x4 lo, hi;
};

template <>
struct Elem<DOPT_BF16> {
    static constexpr int64_t kBytes = 2;
    template <bool NT = false>
    static __device__ __forceinline__ Raw8 load_raw(const void *base, int64_t i) {
        return Raw8{ld16<NT>(static_cast<const uint16_t *>(base) + i), u32x4{0, 0, 0, 0}};
    }
    static __device__ __forceinline__ void unpack(const Raw8 &r, float (&x)[kVec]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __uint_as_float(r.lo[j] << 16);
            x[2 * j + 1] = __uint_as_float(r.lo[j] & 0xffff0000u);
        }
    }
    template <bool NT = false>
    static __device__ __forceinline__ void load8(const void *base, int64_t i, float (&x)[kVec]) {
        unpack(load_raw<NT>(base, i), x);
    }
    static __device__ __forceinline__ uint32_t bits(float x) {
        return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
    }
    static __device__ __forceinline__ void store8(void *base, int64_t i, const float (&x)[kVec]) {
        u32x4 u;
        u[0] = bits(x[0]) | (bits(x[1]) << 16);
        u[1] = bits(x[2]) | (bits(x[3]) << 16);
        u[2] = bits(x[4]) | (bits(x[5]) << 16);
        u[3] = bits(x[6]) | (bits(x[7]) << 16);
        *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(base) + i) = u;
    }
    static __device__ __forceinline__ void store1(void *base, int64_t i, float x) {
        static_cast<uint16_t *>(base)[i] = static_cast<uint16_t>(bits(x));
    }
    // lane's 8 elements of a tile through its resource descriptor
    static __device__ __forceinline__ void bload8(__amdgpu_buffer_rsrc_t r, int32_t lane, float (&x)[kVec]) {
        unpack(Raw8{bld16(r, lane * 16), u32x4{0, 0, 0, 0}}, x);
    }
    static __device__ __forceinline__ float bload1(__amdgpu_buffer_rsrc_t r, int32_t lane, int j) {
        return __uint_as_float(uint32_t(__builtin_amdgcn_raw_buffer_load_b16(r, lane * 16 + j * 2, 0, 0)) << 16);
    }
    static __device__ __forceinline__ void bstore1(__amdgpu_buffer_rsrc_t r, int32_t lane, int j, float x) {
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(bits(x)), r, lane * 16 + j * 2, 0, 0);
    }
    static __device__ __forceinline__ void bstore8(__amdgpu_buffer_rsrc_t r, int32_t lane, const float (&x)[kVec]) {
        u32x4 u;
        u[0] = bits(x[0]) | (bits(x[1]) << 16);
        u[1] = bits(x[2]) | (bits(x[3]) << 16);
        u[2] = bits(x[4]) | (bits(x[5]) << 16);
        u[3] = bits(x[6]) | (bits(x[7]) << 16);
        bst16(r, lane * 16, u);
    }
};

template <>
struct Elem<DOPT_F16> {
    static constexpr int64_t kBytes = 2;
    static __device__ __forceinline__ float up(uint32_t h) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
    }
    template <bool NT = false>
    static __device__ __forceinline__ Raw8 load_raw(const void *base, int64_t i) {
        return Raw8{ld16<NT>(static_cast<const uint16_t *>(base) + i), u32x4{0, 0, 0, 0}};
    }
    static __device__ __forceinline__ void unpack(const Raw8 &r, float (&x)[kVec]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = up(r.lo[j] & 0xffffu);
            x[2 * j + 1] = up(r.lo[j] >> 16);
        }
    }
    template <bool NT = false>
    static __device__ __forceinline__ void load8(const void *base, int64_t i, float (&x)[kVec]) {
        unpack(load_raw<NT>(base, i), x);
    }
    static __device__ __forceinline__ uint32_t bits(float x) {
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
    }
    static __device__ __forceinline__ void store8(void *base, int64_t i, const float (&x)[kVec]) {
        u32x4 u;
        u[0] = bits(x[0]) | (bits(x[1]) << 16);
        u[1] = bits(x[2]) | (bits(x[3]) << 16);
        u[2] = bits(x[4]) | (bits(x[5]) << 16);
        u[3] = bits(x[6]) | (bits(x[7]) << 16);
        *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(base) + i) = u;
    }
    static __device__ __forceinline__ void store1(void *base, int64_t i, float x) {
        static_cast<uint16_t *>(base)[i] = static_cast<uint16_t>(bits(x));
    }
    // lane's 8 elements of a tile through its resource descriptor
    static __device__ __forceinline__ void bload8(__amdgpu_buffer_rsrc_t r, int32_t lane, float (&x)[kVec]) {
        unpack(Raw8{bld16(r, lane * 16), u32x4{0, 0, 0, 0}}, x);
    }
    static __device__ __forceinline__ float bload1(__amdgpu_buffer_rsrc_t r, int32_t lane, int j) {
        return up(__builtin_amdgcn_raw_buffer_load_b16(r, lane * 16 + j * 2, 0, 0));
    }
    static __device__ __forceinline__ void bstore1(__amdgpu_buffer_rsrc_t r, int32_t lane, int j, float x) {
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(bits(x)), r, lane * 16 + j * 2, 0, 0);
    }
    static __device__ __forceinline__ void bstore8(__amdgpu_buffer_rsrc_t r, int32_t lane, const float (&x)[kVec]) {
        u32x4 u;
        u[0] = bits(x[0]) | (bits(x[1]) << 16);
        u[1] = bits(x[2]) | (bits(x[3]) << 16);
        u[2] = bits(x[4]) | (bits(x[5]) << 16);
        u[3] = bits(x[6]) | (bits(x[7]) << 16);
        bst16(r, lane * 16, u);
    }
};

template <bool NT = false>
__device__ __forceinline__ void load8f(const float *base, int64_t i, float (&x)[kVec]) {
    const u32x4 a = ld16<NT>(base + i);
    const u32x4 b = ld16<NT>(base + i + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[j] = __uint_as_float(a[j]);
        x[4 + j] = __uint_as_float(b[j]);
    }
}

__device__ __forceinline__ void store8f(float *base, int64_t i, const float (&x)[kVec]) {
    *reinterpret_cast<f32x4 *>(base + i) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4 *>(base + i + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

// Elem<GD>::store8 with the nontemporal hint (16-byte stores), called by all
// 64 lanes of a wave together, lane l holding elements i .. i+7 with
// i = (the wave's first element) + 8l.  For fp32 each store instruction
// covers one contiguous KiB: lane l writes elements 4l .. 4l+3 and
// 256+4l .. 256+4l+3 of the wave's 512, taken from the lanes that hold them
// (l>>1 and 32 + (l>>1)).  Two stores of a lane's own halves would leave
// every other 16 bytes of each instruction's lines unwritten, and streaming
// stores of such partial lines raised the reduce's write traffic by 11%.
template <int GD>
__device__ __forceinline__ void store8_nt(void *base, int64_t i, const float (&x)[kVec]) {
    if constexpr (GD == DOPT_F32) {
        const int l = static_cast<int>(threadIdx.x & 63);
        const int s0 = l >> 1, s1 = 32 + (l >> 1);
        const bool odd = (l & 1) != 0;
        f32x4 a, c;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float lo0 = __shfl(x[q], s0, 64), hi0 = __shfl(x[4 + q], s0, 64);
            const float lo1 = __shfl(x[q], s1, 64), hi1 = __shfl(x[4 + q], s1, 64);
            a[q] = odd ? hi0 : lo0;
            c[q] = odd ? hi1 : lo1;
        }
        float *w = static_cast<float *>(base) + (i - int64_t(l) * kVec);
        __builtin_nontemporal_store(a, reinterpret_cast<f32x4 *>(w + 4 * l));
        __builtin_nontemporal_store(c, reinterpret_cast<f32x4 *>(w + 256 + 4 * l));
    } else {
        u32x4 u;
        u[0] = Elem<GD>::bits(x[0]) | (Elem<GD>::bits(x[1]) << 16);
        u[1] = Elem<GD>::bits(x[2]) | (Elem<GD>::bits(x[3]) << 16);
        u[2] = Elem<GD>::bits(x[4]) | (Elem<GD>::bits(x[5]) << 16);
        u[3] = Elem<GD>::bits(x[6]) | (Elem<GD>::bits(x[7]) << 16);
        __builtin_nontemporal_store(u, reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(base) + i));
    }
}

__device__ __forceinline__ void bload8f(__amdgpu_buffer_rsrc_t r, int32_t lane, float (&x)[kVec]) {
    const u32x4 a = bld16(r, lane * 32);
    const u32x4 b = bld16(r, lane * 32 + 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[j] = __uint_as_float(a[j]);
        x[4 + j] = __uint_as_float(b[j]);
    }
}

__device__ __forceinline__ void bstore8f(__amdgpu_buffer_rsrc_t r, int32_t lane, const float (&x)[kVec]) {
    bst16(r, lane * 32, u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])});
    bst16(r, lane * 32 + 16,
          u32x4{__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7])});
}

template <>
struct Elem<DOPT_F32> {
    static constexpr int64_t kBytes = 4;
    static __device__ __forceinline__ void bload8(__amdgpu_buffer_rsrc_t r, int32_t lane, float (&x)[kVec]) {
        bload8f(r, lane, x);
    }
    static __device__ __forceinline__ void bstore8(__amdgpu_buffer_rsrc_t r, int32_t lane, const float (&x)[kVec]) {
        bstore8f(r, lane, x);
    }
    static __device__ __forceinline__ float bload1(__amdgpu_buffer_rsrc_t r, int32_t lane, int j) {
        return bld4(r, lane * 32 + j * 4);
    }
    static __device__ __forceinline__ void bstore1(__amdgpu_buffer_rsrc_t r, int32_t lane, int j, float x) {
        bst4(r, lane * 32 + j * 4, x);
    }
    template <bool NT = false>
    static __device__ __forceinline__ Raw8 load_raw(const void *base, int64_t i) {
        const float *f = static_cast<const float *>(base) + i;
        return Raw8{ld16<NT>(f), ld16<NT>(f + 4)};
    }
    static __device__ __forceinline__ void unpack(const Raw8 &r, float (&x)[kVec]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = __uint_as_float(r.lo[j]);
            x[4 + j] = __uint_as_float(r.hi[j]);
        }
    }
    template <bool NT = false>
    static __device__ __forceinline__ void load8(const void *base, int64_t i, float (&x)[kVec]) {
        load8f<NT>(static_cast<const float *>(base), i, x);
    }
    static __device__ __forceinline__ void store8(void *base, int64_t i, const float (&x)[kVec]) {
        store8f(static_cast<float *>(base), i, x);
    }
    static __device__ __forceinline__ void store1(void *base, int64_t i, float x) { static_cast<float *>(base)[i] = x; }
};

// Hyper-group of arena element e of a tile that is not fully covered, or -1
// if e belongs to no param (alignment gap, bucket padding, arena tail).
__device__ __forceinline__ int owner_hgroup(const SegDesc *__restrict__ segs, int32_t first, int32_t cnt, int64_t e) {
    for (int32_t s = first; s < first + cnt; ++s)
        if (segs[s].start <= e && e < segs[s].end) return segs[s].hgroup;
    return -1;
}

// Where the read-only passes (pass 1, the bucket check) put a thread's 8
// elements of a 2048-element tile.  16-bit grads: 8 consecutive elements,
// one 16-byte load.  fp32 grads: 4 consecutive elements in each half of the
// tile, so that each of the thread's two 16-byte loads is part of a 1 KB
// contiguous wave access (streaming fp32 reads measured 7.1 TB/s on MI355X
// this way, 6.0 TB/s with 8 consecutive elements per thread).  Element j of
// the thread sits at tile offset rd_off<GD>(j); unpack() yields them in j
// order.
template <int GD>
__device__ __forceinline__ int64_t rd_off(int j) {
    if (GD == DOPT_F32) return (j < 4 ? 0 : kTile / 2) + int64_t(threadIdx.x) * 4 + (j & 3);
    return int64_t(threadIdx.x) * kVec + j;
}

// The thread's raw grad bytes of the tile starting at element `base`; for
// fp32, `lim` (a multiple of 4 above base) clamps each 4-element load to the
// last 4 elements below it.
template <int GD, bool NT>
__device__ __forceinline__ Raw8 rd_load(const void *grad, int64_t base, int64_t lim) {
    if (GD == DOPT_F32) {
        const float *f = static_cast<const float *>(grad);
        const int64_t a = base + int64_t(threadIdx.x) * 4, b = a + kTile / 2;
        return Raw8{ld16<NT>(f + (a < lim ? a : lim - 4)), ld16<NT>(f + (b < lim ? b : lim - 4))};
    }
    const int64_t i = base + int64_t(threadIdx.x) * kVec;
    return Elem<GD>::template load_raw<NT>(grad, i < lim ? i : lim - kVec);
}

// Bit j set when element rd_off(j) of the tile starting at `base` belongs to
// a param.
template <int GD>
__device__ __forceinline__ uint32_t rd_own_mask(const SegDesc *__restrict__ segs, const TileDesc &td, int64_t base) {
    if (td.seg_count & kTileFull) return 0xffu;
    const int32_t cnt = td.seg_count & kTileCountMask;
    uint32_t mk = 0;
#pragma unroll
    for (int j = 0; j < kVec; ++j)
        if (owner_hgroup(segs, td.seg_first, cnt, base + rd_off<GD>(j)) >= 0) mk |= 1u << j;
    return mk;
}

// ---- finalize: skip, norm, clip, loss scale, step count, AdamW scalars ------
//
// [DO] "三层继承体系": an overflow skips the inner step; clipping uses the
// global norm.  [DS] §3 config: dynamic loss scale starting at 2^16.  Clip
// coefficient max_norm / (norm + 1e-6), applied when below 1; the dynamic
// scale backs off (after `hysteresis` overflows) and grows every
// growth_interval clean steps; AdamW scalars are computed in double and
// rounded once to fp32.  Called by every thread of one workgroup: thread 0
// takes the step decision, then thread h fills the scalars of hyper-group h.
// `cur` is the caller's copy of *st, read at kernel start so that its load
// overlaps the reduction; the new state is written to *st.
__device__ void finalize_block(double sumsq, double zeros, const DevState &cur, DevState *st, StepRec *sr,
                               dopt_stats *out, const FinalizeArgs &a) {
    __shared__ double s_t;
    __shared__ int s_skip;
    if (threadIdx.x == 0) {
        DevState n = cur;
        const int found_inf = isfinite(sumsq) ? 0 : 1;
        const double norm = sqrt(sumsq);
        out->found_inf = found_inf;
        out->skipped = found_inf;
        out->reserved = 0;
        out->sumsq = sumsq;
        out->grad_norm = norm;
        out->num_zeros = static_cast<uint64_t>(zeros);
        out->loss_scale_used = n.scale;
        sr->skip = found_inf;
        sr->inv_scale = n.inv_scale;
        if (n.kind == DOPT_SCALER_DYNAMIC) {
            if (found_inf) {
                n.growth_tracker = 0;
                n.hysteresis_tracker -= 1;
                if (n.hysteresis_tracker <= 0) n.scale = fmax(n.scale * n.backoff_factor, n.min_scale);
            } else {
                n.growth_tracker += 1;
                if (n.growth_tracker == n.growth_interval) {
                    n.growth_tracker = 0;
                    n.hysteresis_tracker = n.hysteresis;
                    n.scale = n.scale * n.growth_factor;
                }
            }
            n.inv_scale = static_cast<float>(1.0 / n.scale);
        }
        out->loss_scale_next = n.scale;
        double clip = 1.0;
        int clip_on = 0;
        if (!found_inf) {
            n.t += 1;
            if (a.max_norm > 0.0) {
                clip = a.max_norm / (norm + 1e-6);
                clip_on = clip < 1.0 ? 1 : 0;
            }
        }
        out->clip_coef = clip;
        out->clip_applied = clip_on;
        sr->clip_on = clip_on;
        sr->clip = clip_on ? static_cast<float>(clip) : 0.0f;
        out->step_count = n.t;
        *st = n;
        s_t = static_cast<double>(n.t);
        s_skip = found_inf;
    }
    __syncthreads();
    const int h = threadIdx.x;
    if (!s_skip && h < a.nh) {
        const dopt_hparams &hp = a.hp[h];
        sr->decay[h] = static_cast<float>(1.0 - hp.lr * hp.weight_decay);
        sr->beta1[h] = static_cast<float>(hp.beta1);
        sr->omb1[h] = static_cast<float>(1.0 - hp.beta1);
        sr->beta2[h] = static_cast<float>(hp.beta2);
        sr->omb2[h] = static_cast<float>(1.0 - hp.beta2);
        sr->eps[h] = static_cast<float>(hp.eps);
        sr->step_size[h] = static_cast<float>(hp.lr / (1.0 - pow(hp.beta1, s_t)));
        sr->sqrt_bc2[h] = static_cast<float>(sqrt(1.0 - pow(hp.beta2, s_t)));
    }
}

__global__ void __launch_bounds__(64) k_finalize(const Record *rec, DevState *st, StepRec *sr, dopt_stats *out,
                                                 FinalizeArgs a) {
    const DevState cur = *st;
    finalize_block(rec->sumsq, rec->zeros, cur, st, sr, out, a);
}

// ---- pass 1: unscale, sum of squares, zero count -----------------------------
//
// [DO] "三层继承体系", second layer (grads to fp32 + unscale + inf/NaN) and
// first layer (grad norm, zero count).  Per element g = fp32(raw) * inv_scale;
// g*g is exact in double, so the double sum of squares is finite exactly when
// every g is finite (its largest possible value, 2^64 * (2^128)^2, is far
// below the double range): the inf/NaN flag is read off the final sum.
//
// Each workgroup writes one partial (double sum of squares, integer zero
// count); k_finish then adds all partials in index order -- the same order
// every run, whatever the device -- so the result is deterministic.

__device__ __forceinline__ void block_sum_store(double acc, unsigned long long z, Partial *__restrict__ dst) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        acc += __shfl_xor(acc, off, 64);
        z += __shfl_xor(z, off, 64);
    }
    __shared__ double s_acc[kBlock / 64];
    __shared__ unsigned long long s_z[kBlock / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        s_acc[wave] = acc;
        s_z[wave] = z;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double a = 0.0;
        unsigned long long zz = 0;
#pragma unroll
        for (int w = 0; w < kBlock / 64; ++w) {
            a += s_acc[w];
            zz += s_z[w];
        }
        dst->sumsq = a;
        dst->zeros = zz;
    }
}

// A workgroup's k-th batch is tiles b + k*G*kStatsUnroll + u*G (b = block,
// G = grid size, u < kStatsUnroll).  Its descriptors come from pass 1's copy
// of the tile table (`groups`), where they are consecutive, so each wave
// reads them with one scalar load: with one load per tile, the scalar-cache
// misses of the ~2000 workgroups of a small window cost MI355X about 3 us.
struct TileGroup {
    TileDesc d[kStatsUnroll];
};

template <int GD, bool NT>
__global__ void __launch_bounds__(kBlock) k_stats(const void *__restrict__ grad, const TileGroup *__restrict__ groups,
                                                 const SegDesc *__restrict__ segs, int64_t n_tiles,
                                                 const DevState *__restrict__ st, Partial *__restrict__ out) {
    const float inv = st->inv_scale;
    double acc = 0.0;
    uint32_t zeros = 0;
    const int64_t G = gridDim.x;
    int64_t q = blockIdx.x;
    for (int64_t t0 = blockIdx.x; t0 < n_tiles; t0 += kStatsUnroll * G, q += G) {
        Raw8 raw[kStatsUnroll];
        // All loads are issued before any is waited for: a tile index past
        // the end is clamped to the last tile (allocated arena memory) and its
        // data ignored (its descriptor is an empty one).
#pragma unroll
        for (int u = 0; u < kStatsUnroll; ++u) {
            const int64_t t = t0 + u * G;
            const int64_t tl = t < n_tiles ? t : n_tiles - 1;
            raw[u] = rd_load<GD, NT>(grad, tl * kTile, n_tiles * kTile);
        }
        const TileGroup tg = groups[q];
        __builtin_amdgcn_sched_barrier(0);  // keep the loads together, ahead of the arithmetic
        // Nearly every batch lies inside one param's shard: no ownership tests
        // there (the descriptors are the same for every thread, so the branch
        // does not diverge).
        bool full = true;
#pragma unroll
        for (int u = 0; u < kStatsUnroll; ++u) full = full && (tg.d[u].seg_count & kTileFull) != 0;
        if (full) {
#pragma unroll
            for (int u = 0; u < kStatsUnroll; ++u) {
                float g[kVec];
                Elem<GD>::unpack(raw[u], g);
#pragma unroll
                for (int j = 0; j < kVec; ++j) {
                    const float x = g[j] * inv;
                    const double xd = static_cast<double>(x);
                    acc = fma(xd, xd, acc);
                    zeros += x == 0.0f ? 1u : 0u;
                }
            }
            continue;
        }
        // The data are consumed without branching on them (an element that is
        // not a shard element adds +0, which leaves the sum unchanged), so the
        // compiler keeps every load ahead of the ownership tests.
#pragma unroll
        for (int u = 0; u < kStatsUnroll; ++u) {
            const uint32_t mk = t0 + u * G < n_tiles ? rd_own_mask<GD>(segs, tg.d[u], (t0 + u * G) * kTile) : 0u;
            float g[kVec];
            Elem<GD>::unpack(raw[u], g);
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                const bool own = (mk >> j) & 1u;
                const float x = g[j] * inv;
                const double xd = own ? static_cast<double>(x) : 0.0;
                acc = fma(xd, xd, acc);
                zeros += (own && x == 0.0f) ? 1u : 0u;
            }
        }
    }
    block_sum_store(acc, zeros, out + blockIdx.x);
}

// ---- fused local fp32 reduce + pass 1 -------------------------------------------
//
// [DP] §3.2 (reduce_scatter_with_fp32_accumulation): the N chunks this rank
// received for each arena slot are added in fp32 in chunk order, starting
// from +0, scaled once, stored in the grad dtype, and the stored value goes
// through pass 1 exactly as in k_stats.  Chunk loads are issued BATCH at a
// time (the adds stay in chunk order); the chunks are read once, so they are
// loaded nontemporally.  Small windows take BATCH = kReduceBatch (latency
// bound: the more loads in flight per thread, the better); large ones
// BATCH = kReduceBatchLarge.  On MI355X with the whole chip busy, 2 loads
// per thread read 64 bf16 chunks 6% faster than 1 and 8 chunks with an fp32
// grad write as fast; 4, or 2 on twice the workgroups, put so many requests
// in flight that the mixed read and write streams slowed down.  NT_GRAD
// stores the reduced grads with the nontemporal hint: large windows, whose
// grads far exceed the last-level cache, reduced 2-4% faster that way (64
// bf16 chunks 6.15-6.17 against 5.93-5.98 TB/s, 8 chunks into fp32 grads
// 5.79-5.83 against 5.58-5.61 with ordinary stores); small ones keep
// ordinary stores, so that pass 2 can still find their grads in the cache.
constexpr int kReduceBatch = 8;
constexpr int kReduceBatchLarge = 2;

template <int GD>
__device__ __forceinline__ float stored_value(float x);
template <>
__device__ __forceinline__ float stored_value<DOPT_F32>(float x) { return x; }
template <>
__device__ __forceinline__ float stored_value<DOPT_BF16>(float x) { return __uint_as_float(Elem<DOPT_BF16>::bits(x) << 16); }
template <>
__device__ __forceinline__ float stored_value<DOPT_F16>(float x) { return Elem<DOPT_F16>::up(Elem<DOPT_F16>::bits(x)); }

template <int WD, int GD, int BATCH, bool NT_GRAD>
__global__ void __launch_bounds__(kBlock) k_reduce_stats(const void *__restrict__ chunks, int64_t stride,
                                                        int32_t n_chunks, float scale, void *__restrict__ grad,
                                                        const TileDesc *__restrict__ tiles,
                                                        const SegDesc *__restrict__ segs, int64_t t_begin,
                                                        int64_t t_end, const DevState *__restrict__ st,
                                                        Partial *__restrict__ out) {
    const float inv = st->inv_scale;
    double acc = 0.0;
    uint32_t zeros = 0;
    for (int64_t t = t_begin + blockIdx.x; t < t_end; t += gridDim.x) {
        const TileDesc td = tiles[t];
        const int64_t i0 = t * kTile + int64_t(threadIdx.x) * kVec;
        float s[kVec];
#pragma unroll
        for (int j = 0; j < kVec; ++j) s[j] = 0.0f;
        // full batches: all BATCH loads issued before the first add
        int32_t c0 = 0;
        for (; c0 + BATCH <= n_chunks; c0 += BATCH) {
            Raw8 raw[BATCH];
#pragma unroll
            for (int b = 0; b < BATCH; ++b)
                raw[b] = Elem<WD>::template load_raw<true>(chunks, int64_t(c0 + b) * stride + i0);
            __builtin_amdgcn_sched_barrier(0);  // keep the loads together, ahead of the adds
#pragma unroll
            for (int b = 0; b < BATCH; ++b) {
                float x[kVec];
                Elem<WD>::unpack(raw[b], x);
#pragma unroll
                for (int j = 0; j < kVec; ++j) s[j] = s[j] + x[j];
            }
        }
        for (; c0 < n_chunks; ++c0) {
            float x[kVec];
            Elem<WD>::template load8<true>(chunks, int64_t(c0) * stride + i0, x);
#pragma unroll
            for (int j = 0; j < kVec; ++j) s[j] = s[j] + x[j];
        }
#pragma unroll
        for (int j = 0; j < kVec; ++j) s[j] = s[j] * scale;
        if constexpr (NT_GRAD)
            store8_nt<GD>(grad, i0, s);
        else
            Elem<GD>::store8(grad, i0, s);
        const int32_t cnt = td.seg_count & kTileCountMask;
        if (cnt == 0) continue;
        const bool full = (td.seg_count & kTileFull) != 0;
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            if (!full && owner_hgroup(segs, td.seg_first, cnt, i0 + j) < 0) continue;
            const float x = stored_value<GD>(s[j]) * inv;
            const double xd = static_cast<double>(x);
            acc = fma(xd, xd, acc);
            zeros += (x == 0.0f) ? 1u : 0u;
        }
    }
    block_sum_store(acc, zeros, out + blockIdx.x);
}

// One workgroup of THREADS: the fixed-order sum of all partials into the
// record, and in the fused form the finalize of the step.  Thread i adds
// partials i, i+THREADS, ... in order (loads issued together, BATCH at a
// time), each wave folds its 64 lanes with a fixed butterfly, and thread 0
// adds the wave sums in order.  Up to kFinishSmall partials (small windows)
// take 256 threads x 8 loads; more (large windows, up to kStatsMaxBlocks per
// buffer) take 1024 threads x 16 loads, one round for 16384 partials.
constexpr int kFinishSmall = 2048;
constexpr int kFinishBatch = 8;  // loads in flight per thread in k_check_finish

template <bool FINALIZE, int THREADS, int BATCH>
__global__ void __launch_bounds__(THREADS) k_finish(const Partial *__restrict__ part, int32_t n,
                                                   Record *__restrict__ rec, DevState *__restrict__ st,
                                                   StepRec *__restrict__ sr, dopt_stats *__restrict__ out,
                                                   FinalizeArgs fa) {
    const DevState cur = *st;  // loaded now, used after the reduction
    double a = 0.0;
    unsigned long long z = 0;
    for (int32_t i0 = threadIdx.x; i0 < n; i0 += BATCH * THREADS) {
        Partial q[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const int32_t i = i0 + j * THREADS;
            q[j] = part[i < n ? i : n - 1];
        }
        __builtin_amdgcn_sched_barrier(0);  // all loads in flight before the first add
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const bool in = i0 + j * THREADS < n;  // a clamped duplicate adds +0
            a += in ? q[j].sumsq : 0.0;
            z += in ? q[j].zeros : 0ull;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        a += __shfl_xor(a, off, 64);
        z += __shfl_xor(z, off, 64);
    }
    __shared__ double s_acc[THREADS / 64];
    __shared__ unsigned long long s_z[THREADS / 64];
    __shared__ double s_tot[2];
    if ((threadIdx.x & 63) == 0) {
        s_acc[threadIdx.x >> 6] = a;
        s_z[threadIdx.x >> 6] = z;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        unsigned long long tz = 0;
#pragma unroll
        for (int w = 0; w < THREADS / 64; ++w) {
            t += s_acc[w];
            tz += s_z[w];
        }
        rec->sumsq = t;
        rec->zeros = static_cast<double>(tz);
        s_tot[0] = t;
        s_tot[1] = static_cast<double>(tz);
    }
    if (FINALIZE) {
        __syncthreads();
        finalize_block(s_tot[0], s_tot[1], cur, st, sr, out, fa);
    }
}

// ---- pre-communication check of whole buckets ---------------------------------
//
// [DP] §2.4 (check_grads of a bucket group) and §3.2 (check_for_nan_in_grad,
// check_for_large_grads), on the raw values of a rank's whole local grad
// buffer: per bucket the double sum of squares (NaN exactly when some grad
// is NaN, since g*g is exact in double and cannot overflow it) and the
// largest |grad| with NaN ignored (infinite exactly when some grad is).
// k_check writes one partial per check tile, keeping kCheckTile / kTile
// loads in flight per thread; k_check_finish adds each bucket's partials in
// tile order (one workgroup per bucket).

struct CheckPartial {
    double sumsq;
    float max_abs, pad;
};
static_assert(sizeof(CheckPartial) == 16, "check partial size");

constexpr int kCheckLoads = static_cast<int>(kCheckTile / kTile);

// Bounds of check tile t from the bucket table alone: the last bucket whose
// first check tile is at most t (a wave-uniform binary search), and the
// tile's place in it.  Equal to the per-tile table the mapper builds.
__device__ __forceinline__ void check_tile_bounds(const CheckBucket *__restrict__ bk, int32_t nb, int64_t t,
                                                  int64_t &start, int64_t &end) {
    int32_t lo = 0, hi = nb - 1;
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (bk[mid].tile_base <= t) lo = mid;
        else hi = mid - 1;
    }
    start = bk[lo].offset + (t - bk[lo].tile_base) * kCheckTile;
    end = bk[lo].offset + bk[lo].numel;
}

// SEARCH: the tile bounds come from the bucket table (check_tile_bounds)
// instead of the per-tile table ct.
template <int GD, bool SEARCH>
__global__ void __launch_bounds__(kBlock) k_check(const void *__restrict__ grad, const CheckTile *__restrict__ ct,
                                                 const CheckBucket *__restrict__ bk, int32_t nb, int64_t n_tiles,
                                                 CheckPartial *__restrict__ part) {
    __shared__ double s_acc[kBlock / 64];
    __shared__ float s_mx[kBlock / 64];
    for (int64_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
        int64_t base, end;
        if (SEARCH) {
            check_tile_bounds(bk, nb, t, base, end);
        } else {
            base = ct[t].start;
            end = ct[t].end;
        }
        Raw8 raw[kCheckLoads];
        // Loads past the bucket end are clamped to its last 8 (16-bit) or 4
        // (fp32) elements (the bucket holds at least 128 elements from the
        // tile start, and its end is a multiple of 128) and their values
        // ignored, so all loads are issued before any is waited for.
#pragma unroll
        for (int u = 0; u < kCheckLoads; ++u) raw[u] = rd_load<GD, true>(grad, base + u * kTile, end);
        __builtin_amdgcn_sched_barrier(0);  // keep the loads together, ahead of the arithmetic
        double acc = 0.0;
        float mx = 0.0f;
#pragma unroll
        for (int u = 0; u < kCheckLoads; ++u) {
            float g[kVec];
            Elem<GD>::unpack(raw[u], g);
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                const bool in = base + u * kTile + rd_off<GD>(j) < end;
                const double xd = in ? static_cast<double>(g[j]) : 0.0;  // +0 leaves the sum unchanged
                acc = fma(xd, xd, acc);
                mx = fmaxf(mx, in ? fabsf(g[j]) : 0.0f);
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            acc += __shfl_xor(acc, off, 64);
            mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        }
        __syncthreads();  // the previous tile's totals have been read
        if ((threadIdx.x & 63) == 0) {
            s_acc[threadIdx.x >> 6] = acc;
            s_mx[threadIdx.x >> 6] = mx;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            double a = 0.0;
            float m = 0.0f;
#pragma unroll
            for (int w = 0; w < kBlock / 64; ++w) {
                a += s_acc[w];
                m = fmaxf(m, s_mx[w]);
            }
            part[t].sumsq = a;
            part[t].max_abs = m;
            part[t].pad = 0.0f;
        }
    }
}

__global__ void __launch_bounds__(kBlock) k_check_finish(const CheckPartial *__restrict__ part,
                                                        const CheckBucket *__restrict__ bk, int32_t n_buckets,
                                                        int64_t n_tiles, double thr,
                                                        dopt_bucket_check *__restrict__ out) {
    const int32_t b = blockIdx.x;
    const int64_t t0 = bk[b].tile_base;
    const int64_t t1 = b + 1 < n_buckets ? bk[b + 1].tile_base : n_tiles;
    double a = 0.0;
    float m = 0.0f;
    for (int64_t i0 = t0 + threadIdx.x; i0 < t1; i0 += kFinishBatch * kBlock) {
        CheckPartial q[kFinishBatch];
#pragma unroll
        for (int j = 0; j < kFinishBatch; ++j) {
            const int64_t i = i0 + int64_t(j) * kBlock;
            q[j] = part[i < t1 ? i : t1 - 1];
        }
        __builtin_amdgcn_sched_barrier(0);  // all loads in flight before the first add
#pragma unroll
        for (int j = 0; j < kFinishBatch; ++j) {
            const bool in = i0 + int64_t(j) * kBlock < t1;  // a clamped duplicate adds +0
            a += in ? q[j].sumsq : 0.0;
            m = fmaxf(m, in ? q[j].max_abs : 0.0f);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        a += __shfl_xor(a, off, 64);
        m = fmaxf(m, __shfl_xor(m, off, 64));
    }
    __shared__ double s_acc[kBlock / 64];
    __shared__ float s_mx[kBlock / 64];
    if ((threadIdx.x & 63) == 0) {
        s_acc[threadIdx.x >> 6] = a;
        s_mx[threadIdx.x >> 6] = m;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double sa = 0.0;
        float sm = 0.0f;
#pragma unroll
        for (int w = 0; w < kBlock / 64; ++w) {
            sa += s_acc[w];
            sm = fmaxf(sm, s_mx[w]);
        }
        out[b].sumsq = sa;
        out[b].max_abs = sm;
        out[b].has_nan = isnan(sa) ? 1 : 0;
        out[b].has_inf = isinf(sm) ? 1 : 0;
        out[b].large = (thr > 0.0 && static_cast<double>(sm) > thr) ? 1 : 0;
    }
}

// Up to kTableBatch bucket-table entries, passed by value (kernel arguments
// hold up to 4 KB), written to dst by one wave.
constexpr int kTableBatch = 160;
struct TableBatch {
    CheckBucket e[kTableBatch];
    int32_t n;
};
static_assert(sizeof(TableBatch) <= 4000, "table batch must fit the kernel argument space");

__global__ void __launch_bounds__(64) k_write_table(CheckBucket *__restrict__ dst, TableBatch tb) {
    for (int i = threadIdx.x; i < tb.n; i += 64) dst[i] = tb.e[i];
}

// ---- pass 2: clip + AdamW + bias correction + write-back --------------------
//
// Inner step on shard_fp32_from_float16 and shard_fp32 ([ZL] §3), then the
// master-to-model copy into the param window ([DO] "分片切片逻辑"; [DS] §2).
// fp32 per element, in this order:
//   g = fp32(raw) * inv_scale;  g = g * clip              (when clipping)
//   p = p * (1 - lr*wd)                                  decoupled decay
//   m = beta1*m + (1-beta1)*g
//   v = beta2*v + (1-beta2)*(g*g)
//   p = p - step_size * (m / (sqrt(v) / sqrt(1-beta2^t) + eps)),
//       step_size = lr / (1-beta1^t)
// and the param window receives p rounded to nearest even (16-bit params) or
// p itself (fp32 params, which are their own master).

struct Hp {
    float decay, b1, omb1, b2, omb2, eps, step, sbc2;
};

__device__ __forceinline__ Hp load_hp(const StepRec *__restrict__ r, int h) {
    return Hp{r->decay[h], r->beta1[h], r->omb1[h], r->beta2[h], r->omb2[h], r->eps[h], r->step_size[h], r->sqrt_bc2[h]};
}

__device__ __forceinline__ void adamw(float raw, float &p, float &m, float &v, float inv, int clip_on, float clip,
                                      const Hp &h) {
    float g = raw * inv;
    if (clip_on) g = g * clip;
    p = p * h.decay;
    m = h.b1 * m + h.omb1 * g;
    v = h.b2 * v + h.omb2 * (g * g);
    const float d = sqrtf(v) / h.sbc2 + h.eps;
    p = p - h.step * (m / d);
}

template <int PD, int GD>
__global__ void __launch_bounds__(kBlock) k_apply(const void *__restrict__ grad, void *__restrict__ param,
                                                 float *__restrict__ master, float *__restrict__ m,
                                                 float *__restrict__ v, const TileDesc *__restrict__ tiles,
                                                 const SegDesc *__restrict__ segs, int64_t n_tiles,
                                                 const StepRec *__restrict__ rec, TileBits tb) {
    const int skip = rec->skip;
    const float inv = rec->inv_scale;
    const int clip_on = rec->clip_on;
    const float clip = rec->clip;
    // One hyper-group's scalars (the bitmap's group, else group 0's) are
    // loaded up front with the other step scalars, so a full tile of that
    // group has no scalar load that waits for its descriptor.
    const int hpre = tb.on ? tb.hg : 0;
    const Hp h0 = load_hp(rec, hpre);
    // A skipped step (overflow) touches no data.  The flag is loaded with
    // the other step scalars, which the first data load waits for anyway.
    if (skip) return;
    float *__restrict__ pm = (PD == DOPT_F32) ? static_cast<float *>(param) : master;
    for (int64_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
        // the data loads and the descriptor (read only for a boundary tile,
        // or when the buffer has no bitmap) are issued before either is
        // waited for (arena memory is allocated for every tile); a tile with
        // no param element goes through the per-element path and stores
        // nothing
        const int64_t tile0 = t * kTile;
        const int32_t lane = threadIdx.x;
        const auto rg = tile_rsrc(static_cast<const char *>(grad) + tile0 * Elem<GD>::kBytes, kTile * Elem<GD>::kBytes);
        const auto rp = tile_rsrc(pm + tile0, kTile * 4);
        const auto rm = tile_rsrc(m + tile0, kTile * 4);
        const auto rv = tile_rsrc(v + tile0, kTile * 4);
        float g[kVec], p[kVec], a[kVec], b[kVec];
        Elem<GD>::bload8(rg, lane, g);
        bload8f(rp, lane, p);
        bload8f(rm, lane, a);
        bload8f(rv, lane, b);
        TileDesc td{0, kTileFull | (hpre << kTileHgShift)};
        if (!tb.on || ((tb.w[t >> 5] >> (t & 31)) & 1u)) td = tiles[t];
        const int32_t cnt = td.seg_count & kTileCountMask;
        if (td.seg_count & kTileFull) {
            const int hg = (td.seg_count >> kTileHgShift) & kTileHgMask;
            const Hp h = hg == hpre ? h0 : load_hp(rec, hg);
#pragma unroll
            for (int j = 0; j < kVec; ++j) adamw(g[j], p[j], a[j], b[j], inv, clip_on, clip, h);
            bstore8f(rp, lane, p);
            bstore8f(rm, lane, a);
            bstore8f(rv, lane, b);
            if (PD != DOPT_F32)
                Elem<PD>::bstore8(tile_rsrc(static_cast<char *>(param) + tile0 * Elem<PD>::kBytes, kTile * Elem<PD>::kBytes),
                                  lane, p);
        } else {
            // A boundary tile: walk the segments that meet it (a wave-uniform
            // loop, so each segment's hyper-group scalars are scalar loads)
            // and update each of the lane's elements that lies in one.  The
            // element is read again from the tile (a cache hit) rather than
            // kept from the loads above, which keeps the kernel's register
            // count, and so its occupancy, that of the full-tile path.
            // Segments are disjoint: each element is updated at most once, and
            // elements of no param are not stored.
            const int64_t e0 = tile0 + int64_t(lane) * kVec;
            const auto rq = tile_rsrc(static_cast<char *>(param) + tile0 * Elem<PD>::kBytes, kTile * Elem<PD>::kBytes);
            for (int32_t sg = td.seg_first; sg < td.seg_first + cnt; ++sg) {
                const int64_t s0 = segs[sg].start, s1 = segs[sg].end;
                const Hp hs = load_hp(rec, segs[sg].hgroup);
#pragma unroll 1
                for (int j = 0; j < kVec; ++j) {
                    if (s0 <= e0 + j && e0 + j < s1) {
                        const int32_t o4 = lane * 32 + j * 4;
                        float pj = bld4(rp, o4), aj = bld4(rm, o4), bj = bld4(rv, o4);
                        adamw(Elem<GD>::bload1(rg, lane, j), pj, aj, bj, inv, clip_on, clip, hs);
                        bst4(rp, o4, pj);
                        bst4(rm, o4, aj);
                        bst4(rv, o4, bj);
                        if (PD != DOPT_F32) Elem<PD>::bstore1(rq, lane, j, pj);
                    }
                }
            }
        }
    }
}

// Pass 2 for a large window (grid-stride) that holds boundary tiles: a tile
// whose segments share one hyper-group updates the 8 elements it already
// holds in registers, as a full tile does, and stores only the owned ones.
// In k_apply a boundary tile walks its elements one at a time, re-reading
// each from the tile; on a grid-stride launch the workgroups that draw such
// tiles fall behind and the launch waits for the slowest (the Llama-3-70B
// rank of N=64 has 381 boundary tiles in 538,283: pass 2 5.18 ms in k_apply,
// 5.10 ms here).  A separate kernel, so that k_apply (every small window, and
// the large ones without boundary tiles) keeps its own code; this one holds
// more registers, capped at 64 so that it never drops below 8 waves per SIMD.
template <int PD, int GD>
__global__ void __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(8)))
k_apply_bnd(const void *__restrict__ grad, void *__restrict__ param, float *__restrict__ master,
            float *__restrict__ m, float *__restrict__ v, const TileDesc *__restrict__ tiles,
            const SegDesc *__restrict__ segs, int64_t n_tiles, const StepRec *__restrict__ rec, TileBits tb) {
    const int skip = rec->skip;
    const float inv = rec->inv_scale;
    const int clip_on = rec->clip_on;
    const float clip = rec->clip;
    const int hpre = tb.on ? tb.hg : 0;
    const Hp h0 = load_hp(rec, hpre);
    if (skip) return;
    float *__restrict__ pm = (PD == DOPT_F32) ? static_cast<float *>(param) : master;
    for (int64_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
        const int64_t tile0 = t * kTile;
        const int32_t lane = threadIdx.x;
        const auto rg = tile_rsrc(static_cast<const char *>(grad) + tile0 * Elem<GD>::kBytes, kTile * Elem<GD>::kBytes);
        const auto rp = tile_rsrc(pm + tile0, kTile * 4);
        const auto rm = tile_rsrc(m + tile0, kTile * 4);
        const auto rv = tile_rsrc(v + tile0, kTile * 4);
        const auto rq = tile_rsrc(static_cast<char *>(param) + tile0 * Elem<PD>::kBytes, kTile * Elem<PD>::kBytes);
        float g[kVec], p[kVec], a[kVec], b[kVec];
        Elem<GD>::bload8(rg, lane, g);
        bload8f(rp, lane, p);
        bload8f(rm, lane, a);
        bload8f(rv, lane, b);
        TileDesc td{0, kTileFull | (hpre << kTileHgShift)};
        if (!tb.on || ((tb.w[t >> 5] >> (t & 31)) & 1u)) td = tiles[t];
        const int32_t cnt = td.seg_count & kTileCountMask;
        const bool full = (td.seg_count & kTileFull) != 0;
        int hg = (td.seg_count >> kTileHgShift) & kTileHgMask;
        uint32_t own = 0xffu;  // the lane's elements that belong to a param
        if (!full) {
            // the segments that meet the tile (disjoint; a wave-uniform loop)
            // give the lane's owned elements
            const int32_t l0 = lane * kVec;  // the lane's first element within the tile
            own = 0;
            hg = cnt > 0 ? segs[td.seg_first].hgroup : hpre;
            bool one_hg = true;
            for (int32_t sg = td.seg_first; sg < td.seg_first + cnt; ++sg) {
                const int32_t lo = static_cast<int32_t>(max(segs[sg].start - tile0, int64_t(0)));
                const int32_t hi = static_cast<int32_t>(min(segs[sg].end - tile0, int64_t(kTile)));
                one_hg = one_hg && segs[sg].hgroup == hg;
#pragma unroll
                for (int j = 0; j < kVec; ++j) own |= (lo <= l0 + j && l0 + j < hi) ? 1u << j : 0u;
            }
            if (!one_hg) {
                // segments of several hyper-groups meet in the tile: each owned
                // element on its own with its segment's scalars, as in k_apply
                const int64_t e0 = tile0 + int64_t(lane) * kVec;
                for (int32_t sg = td.seg_first; sg < td.seg_first + cnt; ++sg) {
                    const int64_t s0 = segs[sg].start, s1 = segs[sg].end;
                    const Hp hs = load_hp(rec, segs[sg].hgroup);
#pragma unroll 1
                    for (int j = 0; j < kVec; ++j) {
                        if (s0 <= e0 + j && e0 + j < s1) {
                            const int32_t o4 = lane * 32 + j * 4;
                            float pj = bld4(rp, o4), aj = bld4(rm, o4), bj = bld4(rv, o4);
                            adamw(Elem<GD>::bload1(rg, lane, j), pj, aj, bj, inv, clip_on, clip, hs);
                            bst4(rp, o4, pj);
                            bst4(rm, o4, aj);
                            bst4(rv, o4, bj);
                            if (PD != DOPT_F32) Elem<PD>::bstore1(rq, lane, j, pj);
                        }
                    }
                }
                continue;
            }
        }
        // one hyper-group: all 8 elements are updated (an element of no param
        // is computed and dropped)
        const Hp h = hg == hpre ? h0 : load_hp(rec, hg);
#pragma unroll
        for (int j = 0; j < kVec; ++j) adamw(g[j], p[j], a[j], b[j], inv, clip_on, clip, h);
        if (full) {
            bstore8f(rp, lane, p);
            bstore8f(rm, lane, a);
            bstore8f(rv, lane, b);
            if (PD != DOPT_F32) Elem<PD>::bstore8(rq, lane, p);
        } else {
            // only the owned elements are stored; the others keep their bytes
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                if ((own >> j) & 1u) {
                    const int32_t o4 = lane * 32 + j * 4;
                    bst4(rp, o4, p[j]);
                    bst4(rm, o4, a[j]);
                    bst4(rv, o4, b[j]);
                    if (PD != DOPT_F32) Elem<PD>::bstore1(rq, lane, j, p[j]);
                }
            }
        }
    }
}

// ---- model-space state export / import -------------------------------------------
//
// Every shard element e of the arena corresponds to export slot
// xoff(seg) + (e - seg.start).  Lane l of a workgroup takes elements
// tile*kTile + j*kBlock + l (j = 0..7), so a wave touches 64 consecutive
// arena slots and, within one segment, 64 consecutive export slots.  The
// fp32 stores carry the nontemporal hint: nothing reads an export soon, and an
// import's arrays are next read by a pass that streams them from HBM.  On
// MI355X the hint took the Llama-3 ranks' import from 5.83-5.85 to 6.02-6.07
// TB/s (70B) and from 6.17-6.25 to 6.30-6.37 TB/s (8B), the export 1-3%.
template <int PD, bool IMPORT>
__global__ void __launch_bounds__(kBlock) k_state_copy(void *__restrict__ param, float *__restrict__ master,
                                                      float *__restrict__ m, float *__restrict__ v,
                                                      const TileDesc *__restrict__ tiles,
                                                      const SegDesc *__restrict__ segs, int64_t t_begin,
                                                      int64_t t_end, float *__restrict__ xm, float *__restrict__ xa,
                                                      float *__restrict__ xv) {
    float *pm = (PD == DOPT_F32) ? static_cast<float *>(param) : master;
    for (int64_t t = t_begin + blockIdx.x; t < t_end; t += gridDim.x) {
        const TileDesc td = tiles[t];
        const int32_t cnt = td.seg_count & kTileCountMask;
        if (cnt == 0) continue;
        if (td.seg_count & kTileFull) {
            // one segment covers the tile: export slot = arena slot + dx; all
            // 24 loads are issued before the first store
            const int64_t dx = segs[td.seg_first].xoff - segs[td.seg_first].start;
            const int64_t e0 = t * kTile + threadIdx.x;
            float a[kVec], b[kVec], c[kVec];
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                const int64_t e = e0 + int64_t(j) * kBlock;
                a[j] = IMPORT ? xm[e + dx] : pm[e];
                b[j] = IMPORT ? xa[e + dx] : m[e];
                c[j] = IMPORT ? xv[e + dx] : v[e];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                const int64_t e = e0 + int64_t(j) * kBlock;
                if (IMPORT) {
                    __builtin_nontemporal_store(a[j], pm + e);
                    __builtin_nontemporal_store(b[j], m + e);
                    __builtin_nontemporal_store(c[j], v + e);
                    if (PD != DOPT_F32) Elem<PD>::store1(param, e, a[j]);
                } else {
                    __builtin_nontemporal_store(a[j], xm + e + dx);
                    __builtin_nontemporal_store(b[j], xa + e + dx);
                    __builtin_nontemporal_store(c[j], xv + e + dx);
                }
            }
            continue;
        }
        // A boundary tile: the segments that meet it (a wave-uniform loop, so
        // their fields are scalar loads) give each of the lane's elements its
        // export offset, and, as in a full tile, every load is issued before
        // the first store.  Elements in no segment (alignment gaps, padding,
        // the arena tail) are neither read nor written.
        const int64_t e0 = t * kTile + threadIdx.x;
        int64_t dx[kVec];
        uint32_t own = 0;
#pragma unroll
        for (int j = 0; j < kVec; ++j) dx[j] = 0;
        for (int32_t sg = td.seg_first; sg < td.seg_first + cnt; ++sg) {
            const int64_t s0 = segs[sg].start, s1 = segs[sg].end, d = segs[sg].xoff - s0;
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                const int64_t e = e0 + int64_t(j) * kBlock;
                if (s0 <= e && e < s1) {
                    dx[j] = d;
                    own |= 1u << j;
                }
            }
        }
        float a[kVec], b[kVec], c[kVec];
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            a[j] = b[j] = c[j] = 0.0f;
            if ((own >> j) & 1u) {
                const int64_t e = e0 + int64_t(j) * kBlock;
                a[j] = IMPORT ? xm[e + dx[j]] : pm[e];
                b[j] = IMPORT ? xa[e + dx[j]] : m[e];
                c[j] = IMPORT ? xv[e + dx[j]] : v[e];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            if ((own >> j) & 1u) {
                const int64_t e = e0 + int64_t(j) * kBlock;
                if (IMPORT) {
                    __builtin_nontemporal_store(a[j], pm + e);
                    __builtin_nontemporal_store(b[j], m + e);
                    __builtin_nontemporal_store(c[j], v + e);
                    if (PD != DOPT_F32) Elem<PD>::store1(param, e, a[j]);
                } else {
                    __builtin_nontemporal_store(a[j], xm + e + dx[j]);
                    __builtin_nontemporal_store(b[j], xa + e + dx[j]);
                    __builtin_nontemporal_store(c[j], xv + e + dx[j]);
                }
            }
        }
    }
}

// ---- state init ---------------------------------------------------------------
// [DO] "分片切片逻辑": the fp32 master is the 16-bit shard converted to float;
// Adam moments start at zero.
template <int PD>
__global__ void __launch_bounds__(kBlock) k_init(const void *__restrict__ param, float *__restrict__ master,
                                                float *__restrict__ m, float *__restrict__ v, int64_t n_tiles) {
    const float z[kVec] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int64_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
        const int64_t i0 = t * kTile + int64_t(threadIdx.x) * kVec;
        if (PD != DOPT_F32) {
            float p[kVec];
            Elem<PD>::load8(param, i0, p);
            store8f(master, i0, p);
        }
        store8f(m, i0, z);
        store8f(v, i0, z);
    }
}

__global__ void k_init_state(DevState *st, StepRec *sr, dopt_stats *stats, Record *rec, InitArgs a) {
    if (threadIdx.x != 0) return;
    *st = a.st;
    StepRec r;
    memset(&r, 0, sizeof r);
    r.skip = 1;
    *sr = r;
    dopt_stats o;
    memset(&o, 0, sizeof o);
    o.loss_scale_next = a.st.scale;
    *stats = o;
    rec->sumsq = 0.0;
    rec->zeros = 0.0;
}

// ---- host side --------------------------------------------------------------

static int hip_check(hipError_t e, const char *what) {
    if (e == hipSuccess) return DOPT_OK;
    return fail(DOPT_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

static int check_launch(const char *what) { return hip_check(hipGetLastError(), what); }

static bool aligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) % DOPT_PTR_ALIGN) == 0; }

static char *ws_ptr(void *ws, int64_t off) { return static_cast<char *>(ws) + off; }

static int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

static int check_bufs(const dopt_layout *L, const dopt_buffer_tensors *bufs, const void *ws, bool need_grad) {
    if (!L || !bufs || !ws) return fail(DOPT_ERR_INVALID, "null layout, tensors or workspace");
    if (!aligned(ws)) return fail(DOPT_ERR_INVALID, "workspace is not 256-byte aligned");
    for (size_t k = 0; k < L->buffers.size(); ++k) {
        const dopt_buffer_tensors &b = bufs[k];
        const bool lowp = L->buffers[k].pd != DOPT_F32;
        const std::string pre = "buffer " + std::to_string(k) + ": ";
        if ((need_grad && !b.grad) || !b.param || !b.exp_avg || !b.exp_avg_sq || (lowp && !b.master))
            return fail(DOPT_ERR_INVALID, pre + "null device pointer");
        if ((need_grad && !aligned(b.grad)) || !aligned(b.param) || !aligned(b.exp_avg) || !aligned(b.exp_avg_sq) ||
            (lowp && !aligned(b.master)))
            return fail(DOPT_ERR_INVALID, pre + "device pointer not 256-byte aligned");
    }
    return DOPT_OK;
}

template <int PD, int GD>
static void launch_apply_dt(bool bnd, dim3 grid, hipStream_t s, const dopt_buffer_tensors &b, const TileDesc *tiles,
                            const SegDesc *segs, int64_t n_tiles, const StepRec *rec, const TileBits &tb) {
    if (bnd)
        k_apply_bnd<PD, GD><<<grid, kBlock, 0, s>>>(b.grad, b.param, b.master, b.exp_avg, b.exp_avg_sq, tiles, segs,
                                                    n_tiles, rec, tb);
    else
        k_apply<PD, GD><<<grid, kBlock, 0, s>>>(b.grad, b.param, b.master, b.exp_avg, b.exp_avg_sq, tiles, segs,
                                                n_tiles, rec, tb);
}

template <int PD>
static void launch_apply_gd(int gd, bool bnd, dim3 grid, hipStream_t s, const dopt_buffer_tensors &b,
                            const TileDesc *tiles, const SegDesc *segs, int64_t n_tiles, const StepRec *rec,
                            const TileBits &tb) {
    switch (gd) {
    case DOPT_BF16:
        launch_apply_dt<PD, DOPT_BF16>(bnd, grid, s, b, tiles, segs, n_tiles, rec, tb);
        break;
    case DOPT_F16:
        launch_apply_dt<PD, DOPT_F16>(bnd, grid, s, b, tiles, segs, n_tiles, rec, tb);
        break;
    default:
        launch_apply_dt<PD, DOPT_F32>(bnd, grid, s, b, tiles, segs, n_tiles, rec, tb);
        break;
    }
}

static int build_finalize_args(const dopt_layout *L, const dopt_hparams *hp, int32_t n_hgroups, double max_grad_norm,
                               FinalizeArgs &a) {
    if (!hp) return fail(DOPT_ERR_INVALID, "null hparams");
    if (n_hgroups < L->max_hgroup + 1 || n_hgroups > DOPT_MAX_HGROUPS)
        return fail(DOPT_ERR_INVALID, "n_hgroups must cover every hgroup of the params (<= DOPT_MAX_HGROUPS)");
    std::memset(&a, 0, sizeof a);
    for (int32_t h = 0; h < n_hgroups; ++h) {
        const dopt_hparams &x = hp[h];
        if (!(x.lr >= 0.0) || !(x.beta1 >= 0.0 && x.beta1 < 1.0) || !(x.beta2 >= 0.0 && x.beta2 < 1.0) ||
            !(x.eps > 0.0) || !(x.weight_decay >= 0.0))
            return fail(DOPT_ERR_INVALID,
                        "hparams " + std::to_string(h) + ": need lr >= 0, 0 <= betas < 1, eps > 0, wd >= 0");
        a.hp[h] = x;
    }
    a.nh = n_hgroups;
    a.max_norm = max_grad_norm;
    return DOPT_OK;
}

// The fixed-order reduction of all pass-1 partials, and the finalize when
// FINALIZE is set.
template <bool FINALIZE>
static int launch_finish(int32_t n_partials, void *ws, hipStream_t stream, const FinalizeArgs &fa) {
    const Partial *part = reinterpret_cast<const Partial *>(ws_ptr(ws, kWsPartials));
    Record *rec = reinterpret_cast<Record *>(ws_ptr(ws, kWsRecord));
    DevState *st = reinterpret_cast<DevState *>(ws_ptr(ws, kWsState));
    StepRec *sr = reinterpret_cast<StepRec *>(ws_ptr(ws, kWsStepRec));
    dopt_stats *out = reinterpret_cast<dopt_stats *>(ws_ptr(ws, kWsStats));
    if (n_partials <= kFinishSmall)
        k_finish<FINALIZE, 256, 8><<<1, 256, 0, stream>>>(part, n_partials, rec, st, sr, out, fa);
    else
        k_finish<FINALIZE, 1024, 16><<<1, 1024, 0, stream>>>(part, n_partials, rec, st, sr, out, fa);
    return check_launch("launch k_finish");
}

// Pass 1 over every buffer, then k_finish.
template <bool FINALIZE>
static int launch_stats(const dopt_layout *L, const dopt_buffer_tensors *bufs, void *ws, hipStream_t stream,
                        const FinalizeArgs &fa) {
    const DevState *st = reinterpret_cast<const DevState *>(ws_ptr(ws, kWsState));
    Partial *part = reinterpret_cast<Partial *>(ws_ptr(ws, kWsPartials));
    for (size_t k = 0; k < L->buffers.size(); ++k) {
        const Buffer &B = L->buffers[k];
        const TileGroup *tiles = reinterpret_cast<const TileGroup *>(ws_ptr(ws, B.ws_stats_tiles));
        const SegDesc *segs = reinterpret_cast<const SegDesc *>(ws_ptr(ws, B.ws_segs));
        const int64_t n_tiles = B.arena_numel / kTile;
        const dim3 grid(B.stats_grid);
        Partial *out = part + B.partial_base;
        // Grad windows larger than the last-level cache are read with
        // nontemporal loads (measured faster for pure streaming reads); smaller
        // ones are read normally so that pass 2's second read can hit the cache.
        const int64_t grad_bytes = B.arena_numel * (B.gd == DOPT_F32 ? 4 : 2);
        const bool nt = grad_bytes > kStreamingReadBytes;
        switch (B.gd) {
        case DOPT_BF16:
            if (nt) k_stats<DOPT_BF16, true><<<grid, kBlock, 0, stream>>>(bufs[k].grad, tiles, segs, n_tiles, st, out);
            else k_stats<DOPT_BF16, false><<<grid, kBlock, 0, stream>>>(bufs[k].grad, tiles, segs, n_tiles, st, out);
            break;
        case DOPT_F16:
            if (nt) k_stats<DOPT_F16, true><<<grid, kBlock, 0, stream>>>(bufs[k].grad, tiles, segs, n_tiles, st, out);
            else k_stats<DOPT_F16, false><<<grid, kBlock, 0, stream>>>(bufs[k].grad, tiles, segs, n_tiles, st, out);
            break;
        default:
            if (nt) k_stats<DOPT_F32, true><<<grid, kBlock, 0, stream>>>(bufs[k].grad, tiles, segs, n_tiles, st, out);
            else k_stats<DOPT_F32, false><<<grid, kBlock, 0, stream>>>(bufs[k].grad, tiles, segs, n_tiles, st, out);
            break;
        }
        int rc = check_launch("launch k_stats");
        if (rc) return rc;
    }
    return launch_finish<FINALIZE>(L->total_partials, ws, stream, fa);
}

// One launch of the fused reduce over tiles [t0, t1) of a buffer; small
// windows (one launch, one tile per workgroup) keep kReduceBatch chunk loads
// in flight per thread, large ones kReduceBatchLarge and store their grads
// with the nontemporal hint.
struct ReduceLaunch {
    dim3 grid;
    const void *chunks;
    int64_t stride;
    int32_t n;
    float scale;
    void *grad;
    const TileDesc *tiles;
    const SegDesc *segs;
    int64_t t0, t1;
    bool small;
    const DevState *st;
    Partial *out;
};

template <int WD, int GD>
static void launch_reduce_dt(const ReduceLaunch &r, hipStream_t s) {
    if (r.small)
        k_reduce_stats<WD, GD, kReduceBatch, false><<<r.grid, kBlock, 0, s>>>(
            r.chunks, r.stride, r.n, r.scale, r.grad, r.tiles, r.segs, r.t0, r.t1, r.st, r.out);
    else
        k_reduce_stats<WD, GD, kReduceBatchLarge, true><<<r.grid, kBlock, 0, s>>>(
            r.chunks, r.stride, r.n, r.scale, r.grad, r.tiles, r.segs, r.t0, r.t1, r.st, r.out);
}

template <int WD>
static void launch_reduce_gd(int gd, const ReduceLaunch &r, hipStream_t s) {
    if (gd == DOPT_BF16)
        launch_reduce_dt<WD, DOPT_BF16>(r, s);
    else if (gd == DOPT_F16)
        launch_reduce_dt<WD, DOPT_F16>(r, s);
    else
        launch_reduce_dt<WD, DOPT_F32>(r, s);
}

// Fused local fp32 reduce + pass 1 over every buffer, then k_finish.
template <bool FINALIZE>
static int launch_reduce(const dopt_layout *L, const dopt_buffer_tensors *bufs, const void *const *chunks,
                         const int64_t *strides, int32_t wd, int32_t n_chunks, float scale, void *ws,
                         hipStream_t stream, const FinalizeArgs &fa) {
    const DevState *st = reinterpret_cast<const DevState *>(ws_ptr(ws, kWsState));
    Partial *part = reinterpret_cast<Partial *>(ws_ptr(ws, kWsPartials));
    for (size_t k = 0; k < L->buffers.size(); ++k) {
        const Buffer &B = L->buffers[k];
        const TileDesc *tiles = reinterpret_cast<const TileDesc *>(ws_ptr(ws, B.ws_tiles));
        const SegDesc *segs = reinterpret_cast<const SegDesc *>(ws_ptr(ws, B.ws_segs));
        const int64_t n_tiles = B.arena_numel / kTile;
        ReduceLaunch r;
        r.grid = dim3(B.reduce_grid);  // one partial per workgroup and launch
        r.chunks = chunks[k];
        r.stride = strides ? strides[k] : B.arena_numel;
        r.n = n_chunks;
        r.scale = scale;
        // the grad arena is this entry point's output (read-only everywhere else)
        r.grad = const_cast<void *>(bufs[k].grad);
        r.tiles = tiles;
        r.segs = segs;
        r.small = n_tiles <= kOneTileGridMax;
        r.st = st;
        for (int32_t l = 0; l < B.reduce_launches; ++l) {
            // every workgroup of every launch writes its partial (idle ones a
            // zero), so the finish reads reduce_grid * reduce_launches of them
            r.t0 = int64_t(l) * kRangeTiles;
            r.t1 = r.small ? n_tiles : std::min(n_tiles, r.t0 + kRangeTiles);
            r.out = part + B.reduce_partial_base + int64_t(l) * B.reduce_grid;
            if (wd == DOPT_BF16)
                launch_reduce_gd<DOPT_BF16>(B.gd, r, stream);
            else if (wd == DOPT_F16)
                launch_reduce_gd<DOPT_F16>(B.gd, r, stream);
            else
                launch_reduce_gd<DOPT_F32>(B.gd, r, stream);
            int rc = check_launch("launch k_reduce_stats");
            if (rc) return rc;
        }
    }
    return launch_finish<FINALIZE>(L->total_reduce_partials, ws, stream, fa);
}

template <bool IMPORT>
static int state_copy(const dopt_layout *L, const dopt_buffer_tensors *bufs, float *xm, float *xa, float *xv,
                      void *ws, hipStream_t stream) {
    int rc = check_bufs(L, bufs, ws, false);
    if (rc != DOPT_OK) return rc;
    if (!xm || !xa || !xv) return fail(DOPT_ERR_INVALID, "null export array");
    for (size_t k = 0; k < L->buffers.size(); ++k) {
        const Buffer &B = L->buffers[k];
        const TileDesc *tiles = reinterpret_cast<const TileDesc *>(ws_ptr(ws, B.ws_tiles));
        const SegDesc *segs = reinterpret_cast<const SegDesc *>(ws_ptr(ws, B.ws_segs));
        const int64_t n_tiles = B.arena_numel / kTile;
        const dim3 grid(B.copy_grid);
        const dopt_buffer_tensors &b = bufs[k];
        // large windows in ranges of kRangeTiles tiles, small ones in one launch
        const int64_t range = n_tiles <= kOneTileGridMax ? n_tiles : kRangeTiles;
        for (int64_t t0 = 0; t0 < n_tiles; t0 += range) {
            const int64_t t1 = std::min(n_tiles, t0 + range);
            if (B.pd == DOPT_BF16)
                k_state_copy<DOPT_BF16, IMPORT><<<grid, kBlock, 0, stream>>>(
                    b.param, b.master, b.exp_avg, b.exp_avg_sq, tiles, segs, t0, t1, xm, xa, xv);
            else if (B.pd == DOPT_F16)
                k_state_copy<DOPT_F16, IMPORT><<<grid, kBlock, 0, stream>>>(
                    b.param, b.master, b.exp_avg, b.exp_avg_sq, tiles, segs, t0, t1, xm, xa, xv);
            else
                k_state_copy<DOPT_F32, IMPORT><<<grid, kBlock, 0, stream>>>(b.param, nullptr, b.exp_avg, b.exp_avg_sq,
                                                                            tiles, segs, t0, t1, xm, xa, xv);
            if ((rc = check_launch("launch k_state_copy"))) return rc;
        }
    }
    return DOPT_OK;
}

// Scan of one buffer's buckets: k_check over its check tiles, then
// k_check_finish per bucket.  SEARCH: tile bounds from the bucket table.
template <bool SEARCH>
static int launch_check(const Buffer &B, const void *grad, const CheckTile *ct, const CheckBucket *bk, int32_t nb,
                        CheckPartial *part, double thr, dopt_bucket_check *out, hipStream_t stream) {
    const dim3 grid(static_cast<uint32_t>(std::min<int64_t>(B.chk_tiles, kCheckMaxBlocks)));
    if (B.gd == DOPT_BF16)
        k_check<DOPT_BF16, SEARCH><<<grid, kBlock, 0, stream>>>(grad, ct, bk, nb, B.chk_tiles, part);
    else if (B.gd == DOPT_F16)
        k_check<DOPT_F16, SEARCH><<<grid, kBlock, 0, stream>>>(grad, ct, bk, nb, B.chk_tiles, part);
    else
        k_check<DOPT_F32, SEARCH><<<grid, kBlock, 0, stream>>>(grad, ct, bk, nb, B.chk_tiles, part);
    int rc = check_launch("launch k_check");
    if (rc) return rc;
    k_check_finish<<<nb, kBlock, 0, stream>>>(part, bk, nb, B.chk_tiles, thr, out);
    return check_launch("launch k_check_finish");
}

// ---- the allocation-free bucket check ------------------------------------------
//
// dopt_check_grads_noalloc keeps its bucket table and its per-check-tile
// partials in `scratch`, a device array of fixed size that every GPU holds
// from module load to process end.  On the host the array's name is only a
// stand-in for the device symbol: its device address is looked up once per
// device (hipGetSymbolAddress, with that device current, on the entry point's
// first call there) and only that address is ever passed to a kernel.
// Calls on one GPU share the array, so calls that overlap in time on one GPU
// race; every call rewrites the table and every partial it reads.
constexpr int64_t kNoAllocScratchBytes = DOPT_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static std::once_flag g_scratch_once[kMaxDevices];
static char *g_scratch_ptr[kMaxDevices];
static hipError_t g_scratch_rc[kMaxDevices];

static int scratch_on_current_device(char **out) {
    int dev = -1;
    int rc = hip_check(hipGetDevice(&dev), "hipGetDevice");
    if (rc) return rc;
    if (dev < 0 || dev >= kMaxDevices) return fail(DOPT_ERR_INVALID, "device index beyond the library's table");
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        g_scratch_rc[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = static_cast<char *>(p);
    });
    if (g_scratch_rc[dev] != hipSuccess)
        return fail(DOPT_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(g_scratch_rc[dev]));
    *out = g_scratch_ptr[dev];
    return DOPT_OK;
}

// A loss scale the step can run with: positive and finite, with a
// reciprocal (the factor every grad is unscaled by, kept in fp32) that is a
// finite nonzero fp32 number.
static bool usable_scale(double s) {
    if (!(s > 0.0) || !std::isfinite(s)) return false;
    const float inv = static_cast<float>(1.0 / s);
    return inv > 0.0f && std::isfinite(inv);
}

}  // namespace dopt

using namespace dopt;

extern "C" {

int dopt_init_state(const dopt_layout *L, const dopt_buffer_tensors *bufs, const dopt_scaler_cfg *sc, void *ws,
                    hipStream_t stream) {
    int rc = check_bufs(L, bufs, ws, false);
    if (rc != DOPT_OK) return rc;
    if (!sc) return fail(DOPT_ERR_INVALID, "null scaler config");
    if (!usable_scale(sc->initial_scale) || (sc->kind != DOPT_SCALER_CONSTANT && sc->kind != DOPT_SCALER_DYNAMIC))
        return fail(DOPT_ERR_INVALID, "scaler: kind must be constant or dynamic, and initial_scale finite and > 0 "
                                      "with a finite nonzero fp32 reciprocal");
    if (sc->kind == DOPT_SCALER_DYNAMIC &&
        (sc->hysteresis < 1 || sc->growth_interval < 1 || !(sc->growth_factor > 1.0) || !std::isfinite(sc->growth_factor) ||
         !(sc->backoff_factor > 0.0) || !(sc->backoff_factor < 1.0) || !usable_scale(sc->min_scale)))
        return fail(DOPT_ERR_INVALID, "dynamic scaler: bad hysteresis, interval or factors");
    for (const Buffer &B : L->buffers) {
        rc = hip_check(hipMemcpyAsync(ws_ptr(ws, B.ws_tiles), B.tiles.data(), B.tiles.size() * sizeof(TileDesc),
                                      hipMemcpyHostToDevice, stream),
                       "copy tile table");
        if (rc) return rc;
        rc = hip_check(hipMemcpyAsync(ws_ptr(ws, B.ws_stats_tiles), B.stats_tiles.data(),
                                      B.stats_tiles.size() * sizeof(TileDesc), hipMemcpyHostToDevice, stream),
                       "copy pass-1 tile table");
        if (rc) return rc;
        if (!B.segs.empty()) {
            rc = hip_check(hipMemcpyAsync(ws_ptr(ws, B.ws_segs), B.segs.data(), B.segs.size() * sizeof(SegDesc),
                                          hipMemcpyHostToDevice, stream),
                           "copy segment table");
            if (rc) return rc;
        }
        rc = hip_check(hipMemcpyAsync(ws_ptr(ws, B.ws_chk), B.chk.data(), B.chk.size() * sizeof(CheckBucket),
                                      hipMemcpyHostToDevice, stream),
                       "copy bucket table");
        if (rc) return rc;
        rc = hip_check(hipMemcpyAsync(ws_ptr(ws, B.ws_chk_tile), B.chk_tile.data(),
                                      B.chk_tile.size() * sizeof(CheckTile), hipMemcpyHostToDevice, stream),
                       "copy check tile table");
        if (rc) return rc;
    }
    for (size_t k = 0; k < L->buffers.size(); ++k) {
        const Buffer &B = L->buffers[k];
        const dopt_buffer_tensors &b = bufs[k];
        const int64_t n_tiles = B.arena_numel / kTile;
        const dim3 grid(B.apply_grid);
        if (B.pd == DOPT_BF16)
            k_init<DOPT_BF16><<<grid, kBlock, 0, stream>>>(b.param, b.master, b.exp_avg, b.exp_avg_sq, n_tiles);
        else if (B.pd == DOPT_F16)
            k_init<DOPT_F16><<<grid, kBlock, 0, stream>>>(b.param, b.master, b.exp_avg, b.exp_avg_sq, n_tiles);
        else
            k_init<DOPT_F32><<<grid, kBlock, 0, stream>>>(b.param, nullptr, b.exp_avg, b.exp_avg_sq, n_tiles);
        if ((rc = check_launch("launch k_init"))) return rc;
    }
    InitArgs a;
    std::memset(&a, 0, sizeof a);
    a.st.scale = sc->initial_scale;
    a.st.growth_factor = sc->growth_factor;
    a.st.backoff_factor = sc->backoff_factor;
    a.st.min_scale = sc->min_scale;
    a.st.t = 0;
    a.st.growth_tracker = 0;
    a.st.hysteresis_tracker = sc->hysteresis;
    a.st.growth_interval = sc->growth_interval;
    a.st.inv_scale = static_cast<float>(1.0 / sc->initial_scale);
    a.st.kind = sc->kind;
    a.st.hysteresis = sc->hysteresis;
    k_init_state<<<1, 64, 0, stream>>>(reinterpret_cast<DevState *>(ws_ptr(ws, kWsState)),
                                       reinterpret_cast<StepRec *>(ws_ptr(ws, kWsStepRec)),
                                       reinterpret_cast<dopt_stats *>(ws_ptr(ws, kWsStats)),
                                       reinterpret_cast<Record *>(ws_ptr(ws, kWsRecord)), a);
    if ((rc = check_launch("launch k_init_state"))) return rc;
    return hip_check(hipStreamSynchronize(stream), "synchronize after init");
}

int dopt_step_stats(const dopt_layout *L, const dopt_buffer_tensors *bufs, void *ws, hipStream_t stream) {
    int rc = check_bufs(L, bufs, ws, true);
    if (rc != DOPT_OK) return rc;
    FinalizeArgs none;
    std::memset(&none, 0, sizeof none);
    return launch_stats<false>(L, bufs, ws, stream, none);
}

int dopt_step_finalize(const dopt_layout *L, const dopt_hparams *hp, int32_t n_hgroups, double max_grad_norm,
                       void *ws, hipStream_t stream) {
    if (!L || !ws) return fail(DOPT_ERR_INVALID, "null layout or workspace");
    FinalizeArgs a;
    int rc = build_finalize_args(L, hp, n_hgroups, max_grad_norm, a);
    if (rc) return rc;
    k_finalize<<<1, 64, 0, stream>>>(reinterpret_cast<const Record *>(ws_ptr(ws, kWsRecord)),
                                     reinterpret_cast<DevState *>(ws_ptr(ws, kWsState)),
                                     reinterpret_cast<StepRec *>(ws_ptr(ws, kWsStepRec)),
                                     reinterpret_cast<dopt_stats *>(ws_ptr(ws, kWsStats)), a);
    return check_launch("launch k_finalize");
}

int dopt_step_prepare(const dopt_layout *L, const dopt_buffer_tensors *bufs, const dopt_hparams *hp,
                      int32_t n_hgroups, double max_grad_norm, void *ws, hipStream_t stream) {
    int rc = check_bufs(L, bufs, ws, true);
    if (rc != DOPT_OK) return rc;
    FinalizeArgs a;
    if ((rc = build_finalize_args(L, hp, n_hgroups, max_grad_norm, a))) return rc;
    return launch_stats<true>(L, bufs, ws, stream, a);
}

int dopt_reduce_prepare(const dopt_layout *L, const dopt_buffer_tensors *bufs, const void *const *chunks,
                        const int64_t *chunk_strides, int32_t wire_dtype, int32_t n_chunks, float scale, const dopt_hparams *hp, int32_t n_hgroups,
                        double max_grad_norm, void *ws, hipStream_t stream) {
    int rc = check_bufs(L, bufs, ws, true);
    if (rc != DOPT_OK) return rc;
    if (L->num_instances != 1)
        return fail(DOPT_ERR_INVALID, "the fp32-accumulating reduce does not support num_instances > 1");
    if (wire_dtype != DOPT_F32 && wire_dtype != DOPT_BF16 && wire_dtype != DOPT_F16)
        return fail(DOPT_ERR_INVALID, "bad wire dtype");
    if (n_chunks != L->dp_size) return fail(DOPT_ERR_INVALID, "n_chunks must equal dp_size (one chunk per rank)");
    if (!chunks) return fail(DOPT_ERR_INVALID, "null chunk array");
    const int64_t wbytes = wire_dtype == DOPT_F32 ? 4 : 2;
    for (size_t k = 0; k < L->buffers.size(); ++k) {
        if (!chunks[k] || !aligned(chunks[k]))
            return fail(DOPT_ERR_INVALID, "buffer " + std::to_string(k) + ": null or unaligned chunk pointer");
        // every chunk starts DOPT_PTR_ALIGN-aligned and holds a whole arena
        if (chunk_strides && (chunk_strides[k] < L->buffers[k].arena_numel || chunk_strides[k] > (int64_t(1) << 40) ||
                              (chunk_strides[k] * wbytes) % DOPT_PTR_ALIGN != 0))
            return fail(DOPT_ERR_INVALID, "buffer " + std::to_string(k) + ": chunk stride " +
                                              std::to_string(chunk_strides[k]) + " below the arena (" +
                                              std::to_string(L->buffers[k].arena_numel) +
                                              " elements), above 2^40 or not a multiple of " +
                                              std::to_string(DOPT_PTR_ALIGN) + " bytes");
        // the n_chunks chunks span less than 2^62 bytes, so every element and
        // byte offset the kernel forms from them fits in 64 bits
        const int64_t stride = chunk_strides ? chunk_strides[k] : L->buffers[k].arena_numel;
        if (stride > (int64_t(1) << 62) / (wbytes * int64_t(n_chunks)))
            return fail(DOPT_ERR_INVALID, "buffer " + std::to_string(k) + ": " + std::to_string(n_chunks) +
                                              " chunks at a stride of " + std::to_string(stride) +
                                              " elements span 2^62 bytes or more");
    }
    FinalizeArgs a;
    std::memset(&a, 0, sizeof a);
    if (hp) {
        if ((rc = build_finalize_args(L, hp, n_hgroups, max_grad_norm, a))) return rc;
        return launch_reduce<true>(L, bufs, chunks, chunk_strides, wire_dtype, n_chunks, scale, ws, stream, a);
    }
    return launch_reduce<false>(L, bufs, chunks, chunk_strides, wire_dtype, n_chunks, scale, ws, stream, a);
}

int dopt_check_grads(const dopt_layout *L, int32_t k, const void *grad, double thr, dopt_bucket_check *out, void *ws,
                     hipStream_t stream) {
    if (!L || !grad || !out || !ws) return fail(DOPT_ERR_INVALID, "null layout, grad buffer, output or workspace");
    if (k < 0 || k >= static_cast<int32_t>(L->buffers.size())) return fail(DOPT_ERR_RANGE, "buffer index");
    if (!aligned(grad) || !aligned(ws) || reinterpret_cast<uintptr_t>(out) % 8 != 0)
        return fail(DOPT_ERR_INVALID, "grad buffer or workspace not 256-byte aligned, or output not 8-byte aligned");
    const Buffer &B = L->buffers[k];
    const CheckBucket *bk = reinterpret_cast<const CheckBucket *>(ws_ptr(ws, B.ws_chk));
    const CheckTile *ct = reinterpret_cast<const CheckTile *>(ws_ptr(ws, B.ws_chk_tile));
    CheckPartial *part = reinterpret_cast<CheckPartial *>(ws_ptr(ws, B.ws_chk_part));
    const int32_t nb = static_cast<int32_t>(B.chk.size());
    return launch_check<false>(B, grad, ct, bk, nb, part, thr, out, stream);
}

int dopt_check_grads_noalloc(const dopt_layout *L, int32_t k, const void *grad, double thr, dopt_bucket_check *out,
                             hipStream_t stream) {
    if (!L || !grad || !out) return fail(DOPT_ERR_INVALID, "null layout, grad buffer or output");
    if (k < 0 || k >= static_cast<int32_t>(L->buffers.size())) return fail(DOPT_ERR_RANGE, "buffer index");
    if (!aligned(grad) || reinterpret_cast<uintptr_t>(out) % 8 != 0)
        return fail(DOPT_ERR_INVALID, "grad buffer not 256-byte aligned, or output not 8-byte aligned");
    const Buffer &B = L->buffers[k];
    const int64_t nb = static_cast<int64_t>(B.chk.size());
    const int64_t tab = align256(nb * static_cast<int64_t>(sizeof(CheckBucket)));
    const int64_t need = tab + B.chk_tiles * static_cast<int64_t>(sizeof(CheckPartial));
    if (need > kNoAllocScratchBytes)
        return fail(DOPT_ERR_INVALID, "buffer " + std::to_string(k) + " needs " + std::to_string(need) +
                                          " bytes of scratch; the static scratch holds " +
                                          std::to_string(kNoAllocScratchBytes) + " (use dopt_check_grads)");
    char *base = nullptr;
    int rc = scratch_on_current_device(&base);
    if (rc) return rc;
    CheckBucket *bk = reinterpret_cast<CheckBucket *>(base);
    CheckPartial *part = reinterpret_cast<CheckPartial *>(base + tab);
    // the bucket table goes into the scratch by kernel arguments (no host
    // copy), kTableBatch entries per launch
    for (int64_t b0 = 0; b0 < nb; b0 += kTableBatch) {
        TableBatch tb;
        tb.n = static_cast<int32_t>(std::min<int64_t>(kTableBatch, nb - b0));
        std::memcpy(tb.e, B.chk.data() + b0, size_t(tb.n) * sizeof(CheckBucket));
        k_write_table<<<1, 64, 0, stream>>>(bk + b0, tb);
        if ((rc = check_launch("launch k_write_table"))) return rc;
    }
    return launch_check<true>(B, grad, nullptr, bk, static_cast<int32_t>(nb), part, thr, out, stream);
}

int dopt_state_export(const dopt_layout *L, const dopt_buffer_tensors *bufs, float *master, float *exp_avg,
                      float *exp_avg_sq, void *ws, hipStream_t stream) {
    return state_copy<false>(L, bufs, master, exp_avg, exp_avg_sq, ws, stream);
}

int dopt_state_import(const dopt_layout *L, const dopt_buffer_tensors *bufs, const float *master,
                      const float *exp_avg, const float *exp_avg_sq, void *ws, hipStream_t stream) {
    return state_copy<true>(L, bufs, const_cast<float *>(master), const_cast<float *>(exp_avg),
                            const_cast<float *>(exp_avg_sq), ws, stream);
}

int dopt_state_scalars_get(const dopt_layout *L, const void *ws, hipStream_t stream, dopt_state_scalars *out) {
    if (!L || !ws || !out) return fail(DOPT_ERR_INVALID, "null layout, workspace or output");
    DevState st;
    int rc = hip_check(hipMemcpyAsync(&st, static_cast<const char *>(ws) + kWsState, sizeof st,
                                      hipMemcpyDeviceToHost, stream),
                       "copy scalar state");
    if (rc) return rc;
    if ((rc = hip_check(hipStreamSynchronize(stream), "synchronize for scalar state"))) return rc;
    out->step_count = st.t;
    out->loss_scale = st.scale;
    out->growth_tracker = st.growth_tracker;
    out->hysteresis_tracker = st.hysteresis_tracker;
    return DOPT_OK;
}

int dopt_state_scalars_set(const dopt_layout *L, void *ws, hipStream_t stream, const dopt_state_scalars *in) {
    if (!L || !ws || !in) return fail(DOPT_ERR_INVALID, "null layout, workspace or input");
    if (!usable_scale(in->loss_scale) || in->step_count < 0)
        return fail(DOPT_ERR_INVALID, "scalar state: loss_scale must be finite and > 0 with a finite nonzero fp32 "
                                      "reciprocal, and step_count >= 0");
    DevState st;
    int rc = hip_check(hipMemcpyAsync(&st, ws_ptr(ws, kWsState), sizeof st, hipMemcpyDeviceToHost, stream),
                       "copy scalar state");
    if (rc) return rc;
    if ((rc = hip_check(hipStreamSynchronize(stream), "synchronize for scalar state"))) return rc;
    st.t = in->step_count;
    st.scale = in->loss_scale;
    st.inv_scale = static_cast<float>(1.0 / in->loss_scale);
    st.growth_tracker = in->growth_tracker;
    st.hysteresis_tracker = in->hysteresis_tracker;
    if ((rc = hip_check(hipMemcpyAsync(ws_ptr(ws, kWsState), &st, sizeof st, hipMemcpyHostToDevice, stream),
                        "write scalar state")))
        return rc;
    return hip_check(hipStreamSynchronize(stream), "synchronize after scalar state");
}

int dopt_step_apply(const dopt_layout *L, const dopt_buffer_tensors *bufs, void *ws, hipStream_t stream) {
    int rc = check_bufs(L, bufs, ws, true);
    if (rc != DOPT_OK) return rc;
    const StepRec *rec = reinterpret_cast<const StepRec *>(ws_ptr(ws, kWsStepRec));
    for (size_t k = 0; k < L->buffers.size(); ++k) {
        const Buffer &B = L->buffers[k];
        const TileDesc *tiles = reinterpret_cast<const TileDesc *>(ws_ptr(ws, B.ws_tiles));
        const SegDesc *segs = reinterpret_cast<const SegDesc *>(ws_ptr(ws, B.ws_segs));
        const int64_t n_tiles = B.arena_numel / kTile;
        const dim3 grid(B.apply_grid);
        switch (B.pd) {
        case DOPT_BF16:
            launch_apply_gd<DOPT_BF16>(B.gd, B.apply_bnd, grid, stream, bufs[k], tiles, segs, n_tiles, rec, B.bits);
            break;
        case DOPT_F16:
            launch_apply_gd<DOPT_F16>(B.gd, B.apply_bnd, grid, stream, bufs[k], tiles, segs, n_tiles, rec, B.bits);
            break;
        default:
            launch_apply_gd<DOPT_F32>(B.gd, B.apply_bnd, grid, stream, bufs[k], tiles, segs, n_tiles, rec, B.bits);
            break;
        }
        if ((rc = check_launch("launch k_apply"))) return rc;
    }
    return DOPT_OK;
}

int dopt_read_stats(const dopt_layout *L, const void *ws, hipStream_t stream, dopt_stats *out) {
    if (!L || !ws || !out) return fail(DOPT_ERR_INVALID, "null layout, workspace or output");
    int rc = hip_check(hipMemcpyAsync(out, static_cast<const char *>(ws) + kWsStats, sizeof(dopt_stats),
                                      hipMemcpyDeviceToHost, stream),
                       "copy stats");
    if (rc) return rc;
    return hip_check(hipStreamSynchronize(stream), "synchronize for stats");
}

int dopt_step(const dopt_layout *L, const dopt_buffer_tensors *bufs, const dopt_hparams *hp, int32_t n_hgroups,
              double max_grad_norm, void *ws, hipStream_t stream, dopt_stats *out) {
    int rc = dopt_step_prepare(L, bufs, hp, n_hgroups, max_grad_norm, ws, stream);
    if (rc) return rc;
    if ((rc = dopt_step_apply(L, bufs, ws, stream))) return rc;
    if (out) return dopt_read_stats(L, ws, stream, out);
    return DOPT_OK;
}

}  // extern "C"
