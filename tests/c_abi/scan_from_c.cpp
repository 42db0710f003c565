// scan_from_c.cpp -- the selective scan driven through its C ABI alone (no
// Python, no PyTorch in the process): host buffers, hipMalloc'd device buffers,
// workspace queries, one training forward and one backward on a stream of our
// own, and the argument checks.  Writes the inputs it generated and every output
// to a binary file for tests/test_gpu_c_abi.py, which compares them with the
// f64 oracle.
//
// usage: scan_from_c <out-file> [batch seqlen d_inner]
// File: int64 batch, seqlen, d_inner, d_state; then float32 arrays in this order:
// x, dt, B, C, z, dy [inputs], A_log, D, dt_bias [params], y, h_last, dx, ddt, dz,
// dB, dC, dA_log, dD, ddt_bias [outputs].
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <math.h>
#include <vector>

#include "ssm_scan.h"

#define HIP_OK(e)                                                              \
    do {                                                                       \
        hipError_t err_ = (e);                                                 \
        if (err_ != hipSuccess) {                                              \
            fprintf(stderr, "%s: %s\n", #e, hipGetErrorString(err_));          \
            exit(3);                                                           \
        }                                                                      \
    } while (0)

// Inputs from a 64-bit LCG (Knuth's MMIX constants), uniform in [-1, 1).
static uint64_t rng_state = 0x2545F4914F6CDD1DULL;
static float uniform() {
    rng_state = rng_state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (float)((double)(rng_state >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0);
}

struct Dev {
    void* p = nullptr;
    size_t n = 0;
    explicit Dev(size_t bytes) : n(bytes) { if (bytes) HIP_OK(hipMalloc(&p, bytes)); }
    ~Dev() { if (p) (void)hipFree(p); }
};

int main(int argc, char** argv) {
    if (argc < 2) {
        fprintf(stderr, "usage: %s <out-file> [batch seqlen d_inner]\n", argv[0]);
        return 2;
    }
    const int64_t Bt = argc > 4 ? atoll(argv[2]) : 2, L = argc > 4 ? atoll(argv[3]) : 300,
                  D = argc > 4 ? atoll(argv[4]) : 96, N = 16;
    ssm_dims dims = {Bt, L, D, N, SSM_F32};

    // argument checks answer before any launch
    ssm_dims bad = dims;
    bad.d_state = 8;
    if (ssm_scan_fwd(&bad, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr) != SSM_E_UNSUPPORTED) {
        fprintf(stderr, "d_state 8 not rejected\n");
        return 1;
    }
    bad = dims;
    bad.seqlen = -1;
    if (ssm_scan_ckpt_bytes(&bad) != 0 || ssm_scan_fwd_workspace_bytes(&bad) != 0) {
        fprintf(stderr, "negative seqlen not rejected\n");
        return 1;
    }

    const size_t act = (size_t)(Bt * L * D), bc = (size_t)(Bt * L * N), st = (size_t)(Bt * D * N);
    std::vector<float> x(act), dt(act), B(bc), C(bc), z(act), dy(act), A_log((size_t)D * N), Dp(D), bias(D);
    for (auto& v : x) v = uniform();
    for (auto& v : dt) v = 0.5f * uniform();
    for (auto& v : B) v = uniform();
    for (auto& v : C) v = uniform();
    for (auto& v : z) v = 2.0f * uniform();
    for (auto& v : dy) v = uniform();
    for (int64_t d = 0; d < D; ++d) {
        for (int64_t n = 0; n < N; ++n) A_log[(size_t)(d * N + n)] = logf((float)(n + 1)) + 0.3f * uniform();
        Dp[(size_t)d] = 1.0f + 0.2f * uniform();
        bias[(size_t)d] = -1.0f + 0.5f * uniform();
    }

    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    Dev dx_(act * 4), ddt_(act * 4), dB_(bc * 4), dC_(bc * 4), dz_(act * 4), dxin(act * 4), ddtin(act * 4),
        dBin(bc * 4), dCin(bc * 4), dzin(act * 4), ddy(act * 4), dA(A_log.size() * 4), dD(D * 4), dbias(D * 4),
        yout(act * 4), dhl(st * 4), gA(A_log.size() * 4), gD(D * 4), gbias(D * 4);
    HIP_OK(hipMemcpy(dxin.p, x.data(), act * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(ddtin.p, dt.data(), act * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dBin.p, B.data(), bc * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dCin.p, C.data(), bc * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dzin.p, z.data(), act * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(ddy.p, dy.data(), act * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dA.p, A_log.data(), A_log.size() * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dD.p, Dp.data(), D * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dbias.p, bias.data(), D * 4, hipMemcpyHostToDevice));

    Dev ckpt(ssm_scan_ckpt_bytes(&dims)), wsf(ssm_scan_fwd_workspace_bytes(&dims)),
        wsb(ssm_scan_bwd_workspace_bytes(&dims));
    ssm_status rc = ssm_scan_fwd(&dims, dxin.p, ddtin.p, dBin.p, dCin.p, dzin.p, (const float*)dA.p,
                                 (const float*)dD.p, (const float*)dbias.p, nullptr, yout.p, (float*)dhl.p,
                                 (float*)ckpt.p, wsf.p, wsf.n, s, nullptr);
    if (rc != SSM_OK) {
        fprintf(stderr, "ssm_scan_fwd: %s\n", ssm_status_str(rc));
        return 1;
    }
    rc = ssm_scan_bwd(&dims, dxin.p, ddtin.p, dBin.p, dCin.p, dzin.p, (const float*)dA.p, (const float*)dD.p,
                      (const float*)dbias.p, nullptr, (const float*)ckpt.p, ddy.p, dx_.p, ddt_.p, dB_.p, dC_.p,
                      dz_.p, (float*)gA.p, (float*)gD.p, (float*)gbias.p, nullptr, wsb.p, wsb.n, s, nullptr);
    if (rc != SSM_OK) {
        fprintf(stderr, "ssm_scan_bwd: %s\n", ssm_status_str(rc));
        return 1;
    }
    HIP_OK(hipStreamSynchronize(s));

    FILE* f = fopen(argv[1], "wb");
    if (!f) {
        perror(argv[1]);
        return 2;
    }
    const int64_t hdr[4] = {Bt, L, D, N};
    fwrite(hdr, sizeof(hdr), 1, f);
    auto put_host = [&](const std::vector<float>& v) { fwrite(v.data(), 4, v.size(), f); };
    auto put_dev = [&](const Dev& d, size_t n) {
        std::vector<float> h(n);
        HIP_OK(hipMemcpy(h.data(), d.p, n * 4, hipMemcpyDeviceToHost));
        fwrite(h.data(), 4, n, f);
    };
    put_host(x); put_host(dt); put_host(B); put_host(C); put_host(z); put_host(dy);
    put_host(A_log); put_host(Dp); put_host(bias);
    put_dev(yout, act); put_dev(dhl, st); put_dev(dx_, act); put_dev(ddt_, act); put_dev(dz_, act);
    put_dev(dB_, bc); put_dev(dC_, bc); put_dev(gA, A_log.size()); put_dev(gD, D); put_dev(gbias, D);
    fclose(f);
    HIP_OK(hipStreamDestroy(s));
    printf("scan_from_c: batch %lld seqlen %lld d_inner %lld ok\n", (long long)Bt, (long long)L, (long long)D);
    return 0;
}
