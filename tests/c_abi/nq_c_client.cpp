// A plain C++ client of libnq.so (no PyTorch, no Python): it allocates with
// hipMalloc, calls the C entry points declared in include/nq.h on its own
// stream, eagerly and inside a captured hipGraph, and writes the outputs
// for the test that compares them with the oracle.
//
//   nq_c_client DIR M D      reads  DIR/x.bin DIR/r.bin (bf16 bits, M x D),
//                                   DIR/gamma.bin (fp32, D)
//                            writes DIR/q.bin DIR/s.bin DIR/ro.bin (eager)
//                                   DIR/qg.bin DIR/sg.bin (graph replay, a
//                                   fresh residual buffer, 3 replays)
//                                   DIR/gq.bin DIR/gs.bin (per-token-group
//                                   FP8 of x, when D % 128 == 0)
//                                   DIR/fq.bin DIR/fs.bin DIR/fro.bin (the
//                                   fused RMSNorm + group-128 FP8, fp32
//                                   scales, when D % 128 == 0)
//                            reads  DIR/beta.bin (fp32, D), DIR/lnscale.bin
//                                   and DIR/nvsg.bin (one fp32 each)
//                            writes DIR/lq.bin (LayerNorm + static e4m3,
//                                   eps 1e-5), DIR/ldq.bin DIR/lds.bin
//                                   (LayerNorm + dynamic e5m2), DIR/nq.bin
//                                   DIR/nsf.bin DIR/nro.bin (residual-add +
//                                   RMSNorm + NVFP4, when D % 16 == 0)
// Exit status 0 on success; a failing call prints its status text.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string>
#include <vector>

#include "nq.h"

#define HIP_OK(x)                                                                                \
    do {                                                                                         \
        hipError_t e_ = (x);                                                                     \
        if (e_ != hipSuccess) {                                                                  \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_));           \
            exit(2);                                                                             \
        }                                                                                        \
    } while (0)
#define NQ_OK_OR_DIE(x)                                                                          \
    do {                                                                                         \
        nq_status s_ = (x);                                                                      \
        if (s_ != NQ_OK) {                                                                       \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, nq_status_string(s_));            \
            exit(3);                                                                             \
        }                                                                                        \
    } while (0)

template <typename T>
static std::vector<T> read_file(const std::string& path, size_t n)
{
    std::vector<T> v(n);
    FILE* f = fopen(path.c_str(), "rb");
    if (!f || fread(v.data(), sizeof(T), n, f) != n) {
        fprintf(stderr, "cannot read %zu elements from %s\n", n, path.c_str());
        exit(4);
    }
    fclose(f);
    return v;
}

template <typename T>
static void write_file(const std::string& path, const std::vector<T>& v)
{
    FILE* f = fopen(path.c_str(), "wb");
    if (!f || fwrite(v.data(), sizeof(T), v.size(), f) != v.size()) {
        fprintf(stderr, "cannot write %s\n", path.c_str());
        exit(4);
    }
    fclose(f);
}

template <typename T>
static T* to_device(const std::vector<T>& h)
{
    T* p = nullptr;
    HIP_OK(hipMalloc(&p, h.size() * sizeof(T)));
    HIP_OK(hipMemcpy(p, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
    return p;
}

template <typename T>
static std::vector<T> to_host(const T* p, size_t n)
{
    std::vector<T> h(n);
    HIP_OK(hipMemcpy(h.data(), p, n * sizeof(T), hipMemcpyDeviceToHost));
    return h;
}

int main(int argc, char** argv)
{
    if (argc != 4) {
        fprintf(stderr, "usage: %s DIR M D\n", argv[0]);
        return 1;
    }
    const std::string dir = argv[1];
    const int64_t M = atoll(argv[2]), D = atoll(argv[3]);
    const size_t n = (size_t)(M * D);
    printf("%s, M=%lld D=%lld\n", nq_version(), (long long)M, (long long)D);

    uint16_t* x = to_device(read_file<uint16_t>(dir + "/x.bin", n));
    uint16_t* r = to_device(read_file<uint16_t>(dir + "/r.bin", n));
    float* gamma = to_device(read_file<float>(dir + "/gamma.bin", (size_t)D));
    uint16_t *ro = nullptr, *ro2 = nullptr;
    uint8_t *q = nullptr, *q2 = nullptr;
    float *s = nullptr, *s2 = nullptr;
    HIP_OK(hipMalloc(&ro, n * 2));
    HIP_OK(hipMalloc(&ro2, n * 2));
    HIP_OK(hipMalloc(&q, n));
    HIP_OK(hipMalloc(&q2, n));
    HIP_OK(hipMalloc(&s, M * 4));
    HIP_OK(hipMalloc(&s2, M * 4));
    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));

    // eager call on the client's stream
    NQ_OK_OR_DIE(nq_fused_add_rmsnorm_quant_fp8(x, D, r, D, ro, D, gamma, 1e-6f, nullptr, q, D, s, nullptr, 0,
                                                M, D, st));
    HIP_OK(hipStreamSynchronize(st));
    write_file(dir + "/q.bin", to_host(q, n));
    write_file(dir + "/s.bin", to_host(s, (size_t)M));
    write_file(dir + "/ro.bin", to_host(ro, n));

    // the same call captured in a graph and replayed
    hipGraph_t g;
    hipGraphExec_t ge;
    HIP_OK(hipStreamBeginCapture(st, hipStreamCaptureModeGlobal));
    NQ_OK_OR_DIE(nq_fused_add_rmsnorm_quant_fp8(x, D, r, D, ro2, D, gamma, 1e-6f, nullptr, q2, D, s2, nullptr, 0,
                                                M, D, st));
    HIP_OK(hipStreamEndCapture(st, &g));
    HIP_OK(hipGraphInstantiate(&ge, g, nullptr, nullptr, 0));
    for (int i = 0; i < 3; ++i) HIP_OK(hipGraphLaunch(ge, st));
    HIP_OK(hipStreamSynchronize(st));
    write_file(dir + "/qg.bin", to_host(q2, n));
    write_file(dir + "/sg.bin", to_host(s2, (size_t)M));

    if (D % 128 == 0) {
        uint8_t* gq = nullptr;
        float* gs = nullptr;
        HIP_OK(hipMalloc(&gq, n));
        HIP_OK(hipMalloc(&gs, (size_t)M * (D / 128) * 4));
        NQ_OK_OR_DIE(nq_per_token_group_quant_fp8(x, D, M, D, 128, NQ_SCALE_FP32, gq, D, gs, st));
        HIP_OK(hipStreamSynchronize(st));
        write_file(dir + "/gq.bin", to_host(gq, n));
        write_file(dir + "/gs.bin", to_host(gs, (size_t)M * (D / 128)));
        HIP_OK(hipFree(gq));
        HIP_OK(hipFree(gs));
    }

    if (D % 128 == 0) {
        uint8_t* fq = nullptr;
        float* fs = nullptr;
        uint16_t* fro = nullptr;
        HIP_OK(hipMalloc(&fq, n));
        HIP_OK(hipMalloc(&fs, (size_t)M * (D / 128) * 4));
        HIP_OK(hipMalloc(&fro, n * 2));
        NQ_OK_OR_DIE(nq_fused_add_rmsnorm_quant_fp8_group(x, D, r, D, fro, D, gamma, 1e-6f, 128, NQ_SCALE_FP32, 0u,
                                                          fq, D, fs, D / 128, nullptr, 0, M, D, st));
        HIP_OK(hipStreamSynchronize(st));
        write_file(dir + "/fq.bin", to_host(fq, n));
        write_file(dir + "/fs.bin", to_host(fs, (size_t)M * (D / 128)));
        write_file(dir + "/fro.bin", to_host(fro, n));
        for (void* p : {(void*)fq, (void*)fs, (void*)fro}) HIP_OK(hipFree(p));
    }

    // LayerNorm: static e4m3 (scale read on the device), then dynamic e5m2
    {
        float* beta = to_device(read_file<float>(dir + "/beta.bin", (size_t)D));
        float* lscale = to_device(read_file<float>(dir + "/lnscale.bin", 1));
        uint8_t *lq = nullptr, *ldq = nullptr;
        float* lds = nullptr;
        HIP_OK(hipMalloc(&lq, n));
        HIP_OK(hipMalloc(&ldq, n));
        HIP_OK(hipMalloc(&lds, M * 4));
        NQ_OK_OR_DIE(nq_layernorm_quant_fp8(x, D, gamma, beta, 1e-5f, lscale, lq, D, M, D, st));
        NQ_OK_OR_DIE(nq_layernorm_quant_fp8_ex(x, D, gamma, beta, 1e-5f, nullptr, NQ_FLAG_E5M2, ldq, D, lds, M, D,
                                               st));
        HIP_OK(hipStreamSynchronize(st));
        write_file(dir + "/lq.bin", to_host(lq, n));
        write_file(dir + "/ldq.bin", to_host(ldq, n));
        write_file(dir + "/lds.bin", to_host(lds, (size_t)M));
        for (void* p : {(void*)beta, (void*)lscale, (void*)lq, (void*)ldq, (void*)lds}) HIP_OK(hipFree(p));
    }

    // residual-add + RMSNorm + NVFP4 (global scale read on the device)
    if (D % 16 == 0) {
        float* sg = to_device(read_file<float>(dir + "/nvsg.bin", 1));
        uint8_t *nqp = nullptr, *nsf = nullptr;
        uint16_t* nro = nullptr;
        HIP_OK(hipMalloc(&nqp, n / 2));
        HIP_OK(hipMalloc(&nsf, n / 16));
        HIP_OK(hipMalloc(&nro, n * 2));
        NQ_OK_OR_DIE(nq_rmsnorm_quant_nvfp4(x, D, r, D, nro, D, gamma, 1e-6f, sg, nqp, D / 2, nsf, D / 16, nullptr, 0,
                                            M, D, st));
        HIP_OK(hipStreamSynchronize(st));
        write_file(dir + "/nq.bin", to_host(nqp, n / 2));
        write_file(dir + "/nsf.bin", to_host(nsf, n / 16));
        write_file(dir + "/nro.bin", to_host(nro, n));
        for (void* p : {(void*)sg, (void*)nqp, (void*)nsf, (void*)nro}) HIP_OK(hipFree(p));
    }

    // a rejected call reports its status and enqueues nothing
    const nq_status bad = nq_fused_add_rmsnorm_quant_fp8(x, D - 1, r, D, ro, D, gamma, 1e-6f, nullptr, q, D, s,
                                                         nullptr, 0, M, D, st);
    printf("stride below the row length -> %s\n", nq_status_string(bad));
    if (bad != NQ_ERR_STRIDE) return 5;

    HIP_OK(hipGraphExecDestroy(ge));
    HIP_OK(hipGraphDestroy(g));
    HIP_OK(hipStreamDestroy(st));
    for (void* p : {(void*)x, (void*)r, (void*)gamma, (void*)ro, (void*)ro2, (void*)q, (void*)q2, (void*)s, (void*)s2})
        HIP_OK(hipFree(p));
    printf("ok\n");
    return 0;
}
