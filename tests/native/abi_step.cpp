// A native consumer of the C ABI in include/dopt.h: no Python, no PyTorch.
// It builds a layout, allocates every device array with hipMalloc, runs the
// steps of an input file on its own HIP stream, and writes the stats and the
// final arenas to an output file for the test to compare with the oracle.
//
//   abi_step layout <in.bin>            print the layout's arena sizes (host only, no GPU)
//   abi_step run <in.bin> <out.bin>     dopt_init_state, then dopt_step per step
//   abi_step reduce <in.bin> <out.bin>  dopt_init_state, then per step the fused
//                                       reduce of the received chunks with the
//                                       finalize (dopt_reduce_prepare), dopt_step_apply
//                                       and dopt_read_stats; after the steps the
//                                       state export and the scalar state
//
// in.bin (little-endian):
//   int32 magic 0x444f5054, n_params, dp_size, dp_rank, steps, n_hgroups
//   int64 bucket_size
//   double max_grad_norm
//   n_hgroups x {double lr, beta1, beta2, eps, weight_decay}
//   n_params  x {int64 numel; int32 param_dtype, grad_dtype, hgroup}
//   per buffer: int64 arena_numel (must equal the layout's)
//   reduce mode only: int32 wire_dtype; float scale
//   per buffer: the initial param arena (arena_numel x param dtype)
//   per step, per buffer: run: the grad arena (arena_numel x grad dtype);
//                         reduce: dp_size chunks back to back (dp_size x arena_numel x wire dtype)
// out.bin:
//   per step: dopt_stats as the ABI defines it
//   per buffer: master (16-bit params only), exp_avg, exp_avg_sq (fp32 arenas), param arena
//   reduce mode only, then: per buffer the grad arena (the last step's reduced grads);
//     int64 state_numel; the exported master, exp_avg, exp_avg_sq (state_numel fp32 each);
//     dopt_state_scalars as the ABI defines it
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "dopt.h"

namespace {

[[noreturn]] void die(const std::string &msg) {
    std::fprintf(stderr, "abi_step: %s\n", msg.c_str());
    std::exit(1);
}

void ck(int rc, const char *what) {
    if (rc != DOPT_OK) die(std::string(what) + " failed (" + std::to_string(rc) + "): " + dopt_last_error());
}

void hk(hipError_t e, const char *what) {
    if (e != hipSuccess) die(std::string(what) + ": " + hipGetErrorString(e));
}

struct Reader {
    FILE *f;
    template <typename T>
    T get() {
        T x;
        if (std::fread(&x, sizeof x, 1, f) != 1) die("input file is short");
        return x;
    }
    void bytes(void *p, size_t n) {
        if (n && std::fread(p, 1, n, f) != n) die("input file is short");
    }
};

int64_t elem_bytes(int32_t dt) { return dt == DOPT_F32 ? 4 : 2; }

struct Input {
    int32_t n_params = 0, N = 0, r = 0, steps = 0, n_hgroups = 0;
    int64_t bucket = 0;
    double max_norm = 0;
    std::vector<dopt_hparams> hp;
    std::vector<dopt_param_desc> params;
};

Input read_header(Reader &rd) {
    Input in;
    if (rd.get<int32_t>() != 0x444f5054) die("bad magic");
    in.n_params = rd.get<int32_t>();
    in.N = rd.get<int32_t>();
    in.r = rd.get<int32_t>();
    in.steps = rd.get<int32_t>();
    in.n_hgroups = rd.get<int32_t>();
    in.bucket = rd.get<int64_t>();
    in.max_norm = rd.get<double>();
    if (in.n_params <= 0 || in.steps < 0 || in.n_hgroups <= 0 || in.n_hgroups > DOPT_MAX_HGROUPS) die("bad header");
    for (int32_t h = 0; h < in.n_hgroups; ++h) {
        dopt_hparams x;
        x.lr = rd.get<double>();
        x.beta1 = rd.get<double>();
        x.beta2 = rd.get<double>();
        x.eps = rd.get<double>();
        x.weight_decay = rd.get<double>();
        in.hp.push_back(x);
    }
    for (int32_t i = 0; i < in.n_params; ++i) {
        dopt_param_desc d;
        std::memset(&d, 0, sizeof d);
        d.numel = rd.get<int64_t>();
        d.param_dtype = rd.get<int32_t>();
        d.grad_dtype = rd.get<int32_t>();
        d.hgroup = rd.get<int32_t>();
        in.params.push_back(d);
    }
    return in;
}

dopt_layout *build(const Input &in) {
    dopt_shard_cfg cfg;
    std::memset(&cfg, 0, sizeof cfg);
    cfg.dp_size = in.N;
    cfg.dp_rank = in.r;
    cfg.bucket_size = in.bucket;
    cfg.num_instances = 1;
    dopt_layout *L = nullptr;
    ck(dopt_build_ranges(in.params.data(), in.n_params, &cfg, &L), "dopt_build_ranges");
    return L;
}

struct DevBuf {
    dopt_buffer_info info;
    void *grad = nullptr, *param = nullptr;
    float *master = nullptr, *m = nullptr, *v = nullptr;
};

}  // namespace

int main(int argc, char **argv) {
    if (argc < 3) die("usage: abi_step layout <in.bin> | abi_step run|reduce <in.bin> <out.bin>");
    const std::string mode = argv[1];
    FILE *f = std::fopen(argv[2], "rb");
    if (!f) die(std::string("cannot open ") + argv[2]);
    Reader rd{f};
    const Input in = read_header(rd);
    dopt_layout *L = build(in);
    const int32_t nb = dopt_layout_num_buffers(L);
    std::vector<DevBuf> bufs(static_cast<size_t>(nb));
    for (int32_t k = 0; k < nb; ++k) ck(dopt_layout_buffer(L, k, &bufs[k].info), "dopt_layout_buffer");
    if (mode == "layout") {
        std::printf("buffers %d workspace %lld\n", nb, static_cast<long long>(dopt_workspace_bytes(L)));
        for (int32_t k = 0; k < nb; ++k)
            std::printf("buffer %d arena_numel %lld shard_numel %lld\n", k,
                        static_cast<long long>(bufs[k].info.arena_numel),
                        static_cast<long long>(bufs[k].info.shard_numel));
        dopt_layout_free(L);
        return 0;
    }
    if ((mode != "run" && mode != "reduce") || argc < 4) die("usage: abi_step run|reduce <in.bin> <out.bin>");
    const bool reduce = mode == "reduce";
    for (int32_t k = 0; k < nb; ++k)
        if (rd.get<int64_t>() != bufs[k].info.arena_numel) die("arena size in the input differs from the layout's");
    int32_t wire = DOPT_BF16;
    float scale = 1.0f;
    if (reduce) {
        wire = rd.get<int32_t>();
        scale = rd.get<float>();
        if (wire != DOPT_F32 && wire != DOPT_BF16 && wire != DOPT_F16) die("bad wire dtype");
    }

    hipStream_t stream;
    hk(hipStreamCreate(&stream), "hipStreamCreate");
    std::vector<dopt_buffer_tensors> t(static_cast<size_t>(nb));
    for (int32_t k = 0; k < nb; ++k) {
        DevBuf &b = bufs[k];
        const int64_t n = b.info.arena_numel;
        hk(hipMalloc(&b.grad, n * elem_bytes(b.info.grad_dtype)), "hipMalloc grad");
        hk(hipMalloc(&b.param, n * elem_bytes(b.info.param_dtype)), "hipMalloc param");
        if (b.info.param_dtype != DOPT_F32) hk(hipMalloc(reinterpret_cast<void **>(&b.master), n * 4), "hipMalloc master");
        hk(hipMalloc(reinterpret_cast<void **>(&b.m), n * 4), "hipMalloc exp_avg");
        hk(hipMalloc(reinterpret_cast<void **>(&b.v), n * 4), "hipMalloc exp_avg_sq");
        std::vector<char> host(static_cast<size_t>(n * elem_bytes(b.info.param_dtype)));
        rd.bytes(host.data(), host.size());
        hk(hipMemcpy(b.param, host.data(), host.size(), hipMemcpyHostToDevice), "copy param");
        t[k] = dopt_buffer_tensors{b.grad, b.param, b.master, b.m, b.v};
    }
    void *ws = nullptr;
    hk(hipMalloc(&ws, static_cast<size_t>(dopt_workspace_bytes(L))), "hipMalloc workspace");
    // reduce mode: one receive buffer per flat buffer, the dp_size chunks back to back
    std::vector<void *> chunks(static_cast<size_t>(nb), nullptr);
    if (reduce)
        for (int32_t k = 0; k < nb; ++k)
            hk(hipMalloc(&chunks[k], static_cast<size_t>(in.N * bufs[k].info.arena_numel * elem_bytes(wire))),
               "hipMalloc chunks");
    dopt_scaler_cfg sc;
    std::memset(&sc, 0, sizeof sc);
    sc.kind = DOPT_SCALER_CONSTANT;
    sc.initial_scale = 1.0;
    ck(dopt_init_state(L, t.data(), &sc, ws, stream), "dopt_init_state");

    FILE *o = std::fopen(argv[3], "wb");
    if (!o) die(std::string("cannot open ") + argv[3]);
    for (int32_t s = 0; s < in.steps; ++s) {
        for (int32_t k = 0; k < nb; ++k) {
            const int64_t n = bufs[k].info.arena_numel;
            const int64_t bytes = reduce ? in.N * n * elem_bytes(wire) : n * elem_bytes(bufs[k].info.grad_dtype);
            std::vector<char> host(static_cast<size_t>(bytes));
            rd.bytes(host.data(), host.size());
            hk(hipMemcpyAsync(reduce ? chunks[k] : bufs[k].grad, host.data(), host.size(), hipMemcpyHostToDevice,
                              stream),
               "copy grad or chunks");
            hk(hipStreamSynchronize(stream), "synchronize after the input copy");
        }
        dopt_stats st;
        if (reduce) {
            ck(dopt_reduce_prepare(L, t.data(), chunks.data(), nullptr, wire, in.N, scale, in.hp.data(), in.n_hgroups,
                                   in.max_norm, ws, stream),
               "dopt_reduce_prepare");
            ck(dopt_step_apply(L, t.data(), ws, stream), "dopt_step_apply");
            ck(dopt_read_stats(L, ws, stream, &st), "dopt_read_stats");
        } else {
            ck(dopt_step(L, t.data(), in.hp.data(), in.n_hgroups, in.max_norm, ws, stream, &st), "dopt_step");
        }
        std::fwrite(&st, sizeof st, 1, o);
    }
    for (int32_t k = 0; k < nb; ++k) {
        const DevBuf &b = bufs[k];
        const int64_t n = b.info.arena_numel;
        std::vector<char> host(static_cast<size_t>(n * 4));
        if (b.master) {
            hk(hipMemcpy(host.data(), b.master, n * 4, hipMemcpyDeviceToHost), "copy master");
            std::fwrite(host.data(), 1, n * 4, o);
        }
        hk(hipMemcpy(host.data(), b.m, n * 4, hipMemcpyDeviceToHost), "copy exp_avg");
        std::fwrite(host.data(), 1, n * 4, o);
        hk(hipMemcpy(host.data(), b.v, n * 4, hipMemcpyDeviceToHost), "copy exp_avg_sq");
        std::fwrite(host.data(), 1, n * 4, o);
        const size_t pb = static_cast<size_t>(n * elem_bytes(b.info.param_dtype));
        hk(hipMemcpy(host.data(), b.param, pb, hipMemcpyDeviceToHost), "copy param");
        std::fwrite(host.data(), 1, pb, o);
    }
    if (reduce) {
        for (int32_t k = 0; k < nb; ++k) {
            const int64_t gb = bufs[k].info.arena_numel * elem_bytes(bufs[k].info.grad_dtype);
            std::vector<char> host(static_cast<size_t>(gb));
            hk(hipMemcpy(host.data(), bufs[k].grad, gb, hipMemcpyDeviceToHost), "copy reduced grad");
            std::fwrite(host.data(), 1, host.size(), o);
        }
        const int64_t sn = dopt_layout_state_numel(L);
        std::fwrite(&sn, sizeof sn, 1, o);
        float *ex[3] = {nullptr, nullptr, nullptr};
        for (float *&e : ex) hk(hipMalloc(reinterpret_cast<void **>(&e), static_cast<size_t>(std::max<int64_t>(sn, 1) * 4)),
                                "hipMalloc export");
        ck(dopt_state_export(L, t.data(), ex[0], ex[1], ex[2], ws, stream), "dopt_state_export");
        hk(hipStreamSynchronize(stream), "synchronize after the export");
        std::vector<float> host(static_cast<size_t>(sn));
        for (float *e : ex) {
            hk(hipMemcpy(host.data(), e, static_cast<size_t>(sn * 4), hipMemcpyDeviceToHost), "copy export");
            std::fwrite(host.data(), 4, host.size(), o);
            hk(hipFree(e), "hipFree");
        }
        dopt_state_scalars sc_out;
        ck(dopt_state_scalars_get(L, ws, stream, &sc_out), "dopt_state_scalars_get");
        std::fwrite(&sc_out, sizeof sc_out, 1, o);
        for (void *c : chunks) hk(hipFree(c), "hipFree");
    }
    std::fclose(o);
    std::fclose(f);
    for (DevBuf &b : bufs) {
        hk(hipFree(b.grad), "hipFree");
        hk(hipFree(b.param), "hipFree");
        if (b.master) hk(hipFree(b.master), "hipFree");
        hk(hipFree(b.m), "hipFree");
        hk(hipFree(b.v), "hipFree");
    }
    hk(hipFree(ws), "hipFree");
    hk(hipStreamDestroy(stream), "hipStreamDestroy");
    dopt_layout_free(L);
    std::printf("ok: %d steps, %d buffers\n", in.steps, nb);
    return 0;
}
