// Streaming roof of the HBM on this GPU: the bandwidth that plain read,
// write and read+write streams reach with hand-written kernels, against which
// the step's passes are judged.  Not part of the library; built by build()
// and run by hand:   tests/native/stream_roof [tiles]   (default 2^17 tiles of
// 2048 elements: 1 GiB per fp32 array).
//
// Streams (every kernel visits tiles t < NT grid-stride and touches elements
// t*2048 .. t*2048+2047 of each array only):
//   read      one fp32 array read (nontemporal loads, 8 x 16 B in flight per lane;
//             a batch's 4 tiles past the end repeat the last tile, so the rate
//             is slightly understated when NT is not a multiple of 4 x grid)
//   write     one fp32 array written
//   copy      one fp32 array read, another written
//   3r3w-out  three fp32 arrays read, three others written
//   3r3w-in   three fp32 arrays read and written in place
//   pass2     three fp32 arrays read and written in place, plus a 16-bit array
//             read and another written (the shape of the step's second pass)
// Lane mappings for the fp32 arrays:
//   m8   8 consecutive elements per lane (two 16-byte accesses 16 bytes apart)
//   m4h  4 consecutive elements per lane in each half of the tile (each
//        16-byte instruction covers 1 KB contiguous per wave)
// Then an XCD placement check: a copy in which chunk c of the buffer is given
// only to the workgroups of XCD (c + s) mod 8 (workgroup i runs on XCD i mod 8,
// which the program checks with the XCC id register), for every shift s.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef unsigned int u2 __attribute__((ext_vector_type(2)));

#define CK(x)                                                                                   \
    do {                                                                                        \
        hipError_t e_ = (x);                                                                    \
        if (e_ != hipSuccess) {                                                                 \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);          \
            std::exit(1);                                                                       \
        }                                                                                       \
    } while (0)

constexpr int kTile = 2048;

struct Arrays {
    float *in[3];
    float *out[3];
    const uint16_t *h_in;
    uint16_t *h_out;
};

__device__ __forceinline__ float upd(float x, int k) { return x * 0.999f + static_cast<float>(k); }

// element offsets of a lane's 8 elements: m8 -> 8*l + j; m4h -> (j < 4 ? 4*l + j : 1024 + 4*l + j - 4)
template <int MAP>
__device__ __forceinline__ void ld8(const float *p, int l, float (&x)[8]) {
    const f4 a = *reinterpret_cast<const f4 *>(p + (MAP == 0 ? 8 * l : 4 * l));
    const f4 b = *reinterpret_cast<const f4 *>(p + (MAP == 0 ? 8 * l + 4 : 1024 + 4 * l));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[j] = a[j];
        x[4 + j] = b[j];
    }
}
template <int MAP>
__device__ __forceinline__ void st8(float *p, int l, const float (&x)[8]) {
    *reinterpret_cast<f4 *>(p + (MAP == 0 ? 8 * l : 4 * l)) = f4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f4 *>(p + (MAP == 0 ? 8 * l + 4 : 1024 + 4 * l)) = f4{x[4], x[5], x[6], x[7]};
}
template <int MAP>
__device__ __forceinline__ void ld8h(const uint16_t *p, int l, float (&x)[8]) {
    if (MAP == 0) {
        const u4 r = *reinterpret_cast<const u4 *>(p + 8 * l);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __uint_as_float(r[j] << 16);
            x[2 * j + 1] = __uint_as_float(r[j] & 0xffff0000u);
        }
    } else {
        const u2 r0 = *reinterpret_cast<const u2 *>(p + 4 * l);
        const u2 r1 = *reinterpret_cast<const u2 *>(p + 1024 + 4 * l);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            x[2 * j] = __uint_as_float(r0[j] << 16);
            x[2 * j + 1] = __uint_as_float(r0[j] & 0xffff0000u);
            x[4 + 2 * j] = __uint_as_float(r1[j] << 16);
            x[5 + 2 * j] = __uint_as_float(r1[j] & 0xffff0000u);
        }
    }
}
template <int MAP>
__device__ __forceinline__ void st8h(uint16_t *p, int l, const float (&x)[8]) {
    u4 u;
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = (__float_as_uint(x[2 * j]) >> 16) | (__float_as_uint(x[2 * j + 1]) & 0xffff0000u);
    if (MAP == 0) {
        *reinterpret_cast<u4 *>(p + 8 * l) = u;
    } else {
        *reinterpret_cast<u2 *>(p + 4 * l) = u2{u[0], u[1]};
        *reinterpret_cast<u2 *>(p + 1024 + 4 * l) = u2{u[2], u[3]};
    }
}

// KIND: 0 copy, 1 3r3w-out, 2 3r3w-in, 3 pass2, 4 write
template <int KIND, int MAP>
__global__ void __launch_bounds__(256) k_stream(Arrays A, int64_t NT) {
    const int l = threadIdx.x;
    constexpr int NS = KIND == 0 || KIND == 4 ? 1 : 3;
    for (int64_t t = blockIdx.x; t < NT; t += gridDim.x) {
        const int64_t base = t * kTile;
        float x[NS][8], h[8];
        if (KIND != 4) {
#pragma unroll
            for (int s = 0; s < NS; ++s) ld8<MAP>(A.in[s] + base, l, x[s]);
            if (KIND == 3) ld8h<MAP>(A.h_in + base, l, h);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) x[0][j] = static_cast<float>(t + j);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j) x[s][j] = upd(x[s][j], s) + (KIND == 3 ? h[j] : 0.0f);
        float *const *dst = (KIND == 2 || KIND == 3) ? A.in : A.out;
#pragma unroll
        for (int s = 0; s < NS; ++s) st8<MAP>(dst[s] + base, l, x[s]);
        if (KIND == 3) st8h<MAP>(A.h_out + base, l, x[0]);
    }
}

// one fp32 array read with nontemporal loads: 4 tiles per batch, both halves
// of each (8 x 16 B in flight per lane)
__global__ void __launch_bounds__(256) k_read(const float *__restrict__ in, int64_t NT, float *__restrict__ sink) {
    const int l = threadIdx.x;
    float acc = 0.0f;
    for (int64_t t0 = blockIdx.x; t0 < NT; t0 += 4 * int64_t(gridDim.x)) {
        f4 v[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t t = t0 + u * int64_t(gridDim.x);
            const int64_t tl = t < NT ? t : NT - 1;
            const float *p = in + tl * kTile + 4 * l;
            v[2 * u] = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(p));
            v[2 * u + 1] = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(p + 1024));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u][0] + v[u][3];
    }
    sink[blockIdx.x * 256 + l] = acc;
}

__global__ void k_xcc(int *out) {
    if (threadIdx.x == 0) {
        unsigned v;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
        out[blockIdx.x] = static_cast<int>(v & 0xf);
    }
}

// copy of chunks of g16 16-byte words; chunk c goes to XCD (c + shift) % 8
// (shift < 0: every workgroup takes every grid-th chunk, no placement)
__global__ void __launch_bounds__(256) k_xcd_copy(const u4 *__restrict__ src, u4 *__restrict__ dst,
                                                  int64_t n_chunks, int64_t g16, int shift) {
    if (shift < 0) {
        for (int64_t c = blockIdx.x; c < n_chunks; c += gridDim.x)
            for (int64_t i = threadIdx.x; i < g16; i += 256) dst[c * g16 + i] = src[c * g16 + i];
        return;
    }
    const int64_t r = ((blockIdx.x & 7) - shift + 8) & 7;
    const int64_t per_xcd = gridDim.x >> 3;
    for (int64_t j = blockIdx.x >> 3; 8 * j + r < n_chunks; j += per_xcd) {
        const int64_t c = 8 * j + r;
        for (int64_t i = threadIdx.x; i < g16; i += 256) dst[c * g16 + i] = src[c * g16 + i];
    }
}

template <typename F>
float time_ms(F launch) {
    hipEvent_t a, b;
    CK(hipEventCreate(&a));
    CK(hipEventCreate(&b));
    launch();
    launch();
    CK(hipGetLastError());
    CK(hipDeviceSynchronize());
    const int reps = 10;
    CK(hipEventRecord(a));
    for (int i = 0; i < reps; ++i) launch();
    CK(hipEventRecord(b));
    CK(hipEventSynchronize(b));
    float ms = 0.0f;
    CK(hipEventElapsedTime(&ms, a, b));
    CK(hipEventDestroy(a));
    CK(hipEventDestroy(b));
    return ms / reps;
}

template <int KIND, int MAP>
void stream_row(const char *name, const char *map, const Arrays &A, int64_t NT, const int *grids, int ng) {
    const double n = double(NT) * kTile;
    const double bytes = KIND == 0 ? 8 * n : KIND == 4 ? 4 * n : KIND == 3 ? 28 * n : 24 * n;
    std::printf("| %s | %s |", name, map);
    for (int i = 0; i < ng; ++i) {
        const int g = grids[i];
        const float ms = time_ms([&] { k_stream<KIND, MAP><<<g, 256>>>(A, NT); });
        std::printf(" %.0f |", bytes / (ms * 1e-3) / 1e9);
    }
    std::printf("\n");
    std::fflush(stdout);
}

int main(int argc, char **argv) {
    const int64_t NT = argc > 1 ? std::atoll(argv[1]) : (int64_t(1) << 17);
    if (NT < 1 || NT > (int64_t(1) << 20)) {
        std::printf("tiles must be in [1, 2^20]\n");
        return 1;
    }
    const int64_t n = NT * kTile;
    Arrays A;
    for (int s = 0; s < 3; ++s) {
        CK(hipMalloc(&A.in[s], n * 4));
        CK(hipMalloc(&A.out[s], n * 4));
        CK(hipMemset(A.in[s], 0, n * 4));
        CK(hipMemset(A.out[s], 0, n * 4));
    }
    uint16_t *hi, *ho;
    CK(hipMalloc(&hi, n * 2));
    CK(hipMalloc(&ho, n * 2));
    CK(hipMemset(hi, 0, n * 2));
    CK(hipMemset(ho, 0, n * 2));
    A.h_in = hi;
    A.h_out = ho;
    const int grids[] = {256, 512, 1024, 2048};
    const int ng = 4;
    float *sink;
    CK(hipMalloc(&sink, size_t(16384) * 256 * 4));

    std::printf("%lld elements per array (%.2f GiB fp32); GB/s by workgroups per launch\n\n", (long long)n,
                n * 4.0 / (1 << 30));
    std::printf("| stream | lanes | 256 | 512 | 1024 | 2048 |\n|---|---|---|---|---|---|\n");
    {
        std::printf("| read | m4h, nontemporal |");
        for (int i = 0; i < ng; ++i) {
            const int g = grids[i];
            const float ms = time_ms([&] { k_read<<<g, 256>>>(A.in[0], NT, sink); });
            std::printf(" %.0f |", 4.0 * n / (ms * 1e-3) / 1e9);
        }
        std::printf("\n");
    }
    stream_row<4, 0>("write", "m8", A, NT, grids, ng);
    stream_row<4, 1>("write", "m4h", A, NT, grids, ng);
    stream_row<0, 0>("copy", "m8", A, NT, grids, ng);
    stream_row<0, 1>("copy", "m4h", A, NT, grids, ng);
    stream_row<1, 0>("3r3w-out", "m8", A, NT, grids, ng);
    stream_row<1, 1>("3r3w-out", "m4h", A, NT, grids, ng);
    stream_row<2, 0>("3r3w-in", "m8", A, NT, grids, ng);
    stream_row<2, 1>("3r3w-in", "m4h", A, NT, grids, ng);
    stream_row<3, 0>("pass2", "m8", A, NT, grids, ng);
    stream_row<3, 1>("pass2", "m4h", A, NT, grids, ng);

    // XCD placement
    const int xg = 2048;
    int *xcc;
    CK(hipMalloc(&xcc, xg * sizeof(int)));
    k_xcc<<<xg, 64>>>(xcc);
    CK(hipDeviceSynchronize());
    int *h = static_cast<int *>(std::malloc(xg * sizeof(int)));
    CK(hipMemcpy(h, xcc, xg * sizeof(int), hipMemcpyDeviceToHost));
    int match = 0;
    for (int i = 0; i < xg; ++i) match += h[i] == (i & 7);
    std::printf("\nXCC id == workgroup index mod 8 for %d of %d workgroups\n\n", match, xg);
    std::printf("| chunk bytes | no placement | s=0 | s=1 | s=2 | s=3 | s=4 | s=5 | s=6 | s=7 |\n");
    std::printf("|---|---|---|---|---|---|---|---|---|---|\n");
    const u4 *src = reinterpret_cast<const u4 *>(A.in[0]);
    u4 *dst = reinterpret_cast<u4 *>(A.out[0]);
    const int64_t bytes = n * 4;
    const int64_t sizes[] = {4096, 16384, 65536, 2097152};
    for (int64_t G : sizes) {
        if (bytes % G) continue;
        const int64_t nc = bytes / G, g16 = G / 16;
        std::printf("| %lld |", (long long)G);
        for (int s = -1; s < 8; ++s) {
            const float ms = time_ms([&] { k_xcd_copy<<<xg, 256>>>(src, dst, nc, g16, s); });
            std::printf(" %.0f |", 2.0 * bytes / (ms * 1e-3) / 1e9);
        }
        std::printf("\n");
        std::fflush(stdout);
    }
    std::free(h);
    CK(hipFree(xcc));
    CK(hipFree(sink));
    for (int s = 0; s < 3; ++s) {
        CK(hipFree(A.in[s]));
        CK(hipFree(A.out[s]));
    }
    CK(hipFree(hi));
    CK(hipFree(ho));
    std::printf("\ndone\n");
    return 0;
}
